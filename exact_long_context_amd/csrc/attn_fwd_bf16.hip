// Ring-ordered exact attention forward, bf16 inputs, d = 128, for gfx950.
//
// Workgroup = 8 waves, two per SIMD.  Each wave owns 32 query rows of one
// query head for the whole walk over the KV tiles and keeps on chip:
//   * its Q tile as MFMA B operands (32 rows x 128 bf16 = 32 VGPRs),
//   * the transposed output accumulator O^T (128 x 32 fp32 = 64 registers),
//   * the reference max m, the exact running max and a per-lane partial l.
// K and V tiles of 64 keys are staged through LDS and read by all 8 waves;
// with grouped-query attention the waves are the query heads of one KV head
// (4 heads x 64 rows), so each K/V byte fetched serves 4 heads.
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
// Ping-pong schedule.  Waves 0-3 (group A) and 4-7 (group B) share the SIMDs
// pairwise.  Each wave alternates two kinds of slot, with group B one slot
// behind group A (one workgroup barrier per iteration, after the second slot;
// within an iteration the hardware arbitrates between the pair):
//   matrix slot : S^T of tile n and O^T += V^T P^T of tile n-1 (32 MFMA,
//                 operand reads issued ahead of use)
//   vector slot : mask / max / exponentials / row sum of the tile whose S^T
//                 it holds
// so while one wave of a SIMD runs its matrix slot the other runs its vector
// slot, and the matrix core and the vector ALU work at the same time.
// Staging: buffer loads that write LDS directly (no registers, no LDS store
// instructions); iteration n fills K buffer (n+1) % 2 with K(n+1) and V buffer
// n % 2 with V(n), issued at the start of the iteration and waited for at its
// end (64 KiB of LDS for the tiles, 16 KiB for the run table).
//
// Layout tricks:
//   * S is computed transposed (keys x queries): one query per lane, 32 keys
//     per lane, so the row max is in-lane plus one half-wave exchange and the
//     row sum needs no exchange until the end.
//   * The K rows fed to the QK MFMA are permuted (bits 2 and 3 of the row index
//     swapped) so that the 8 keys a lane holds per PV MFMA are 8 consecutive
//     keys.
//   * V stays row-major in LDS; the V^T operand comes from transposing LDS
//     reads (ds_read_b64_tr_b16), so V needs no register transposes.
//   * K and V load through buffer resources bounded by the KV segment: rows
//     past the segment end read as zero, with no per-row branches.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "fwd_common.h"
#include "kernels.h"
#include "schedule.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 128;
constexpr int BN = 64;           // keys per tile
constexpr int WAVE_ROWS = 32;    // query rows per wave
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int ROWB = D * 2;        // bytes of one K or V row
constexpr int KTILE = BN * ROWB;   // 16 KiB
constexpr int VTILE = BN * ROWB;   // 16 KiB
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float RESCALE_SLACK = 8.0f;  // log2 units

// K tile in LDS: blocks of 16 rows; inside a block, 16-byte chunk c of all 16
// rows comes before chunk c + 1.  A K operand read (16 rows at one chunk per
// 16 lanes) then covers 256 contiguous bytes, and the 16-key steps of a read
// sequence differ by constants.  A 1 KiB staging block holds 4 chunks of 16
// rows (64 bytes of each global row).
__device__ __forceinline__ int k_pos(int row, int chunk) { return (row >> 4) * 4096 + chunk * 256 + (row & 15) * 16; }
// V tile in LDS: row-major (one 256-byte row per key), 16-byte chunk c of key
// row r stored at c ^ 4 (r % 4).  The V^T operand comes from two transposing
// reads (ds_read_b64_tr_b16), each over 4 consecutive keys x 16 dv per
// 16 lanes; the swizzle puts the four 64-byte pieces of those keys on
// different banks.  Staging writes whole rows: byte key * ROWB + 16 (c ^ 4 (key % 4)).
// Row of the K tile that feeds MFMA row i of a 32-key block.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Combine a value with the one held by lane l ^ 32.  v_permlane32_swap
// exchanges the upper half of one operand with the lower half of the other,
// so for every lane its two results are x[l] and x[l ^ 32] (in an order that
// depends on the half); max and sum are symmetric in them.
__device__ __forceinline__ float max_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One run = the key rows of one KV segment that a workgroup visits: ring step
// t, KV segment sb.  The table of all runs is built once per workgroup in LDS
// (rows of the KV buffer, segment length, causal offset, keys to visit) so
// that the per-tile bookkeeping is a few scalar adds.
constexpr int MAX_RUNS = BF16_MAX_RUNS;
struct Run {
  int32_t kv_row;  // buffer row of the segment's row 0
  int32_t kv_len;  // rows in the segment
  int32_t delta;   // causal offset, clamped to [-(2^30), 2^30]
  int32_t k_end;   // keys to visit (0: nothing in this run)
};

__device__ __forceinline__ Run make_run(const FwdArgs& a, const QGeom& qg, int32_t p_hi, int32_t r) {
  Run e;
  int64_t dl = 0;
  if (a.mode == MODE_CHUNK) {
    e.kv_row = 0;
    e.kv_len = a.lk;
    dl = a.delta;
  } else {
    // MODE_RING: run r is segment r % nseg of step r / nseg; MODE_STEP: the
    // segments of the one step, in a buffer that holds only its KV chunk
    const int32_t nseg = num_segments(a.layout);
    const bool one_step = a.mode == MODE_STEP;
    const int32_t t = one_step ? a.step : (nseg == 2 ? (r >> 1) : r);
    const int32_t sb = nseg == 2 ? (r & 1) : 0;
    const int32_t j = ring_kv_chunk(qg.qchunk, t, a.n_chunks);
    const Segment ks = segment_l(a.layout, a.lq, a.n_chunks, j, sb);
    e.kv_row = (one_step ? 0 : j * a.lq) + ks.row0;
    e.kv_len = ks.len;
    dl = a.causal ? pair_delta(qg.seg, ks) : 0;
  }
  int64_t end = e.kv_len;
  if (a.causal) {
    const int64_t x = (int64_t)p_hi + dl + 1;
    end = x < 0 ? 0 : (x < end ? x : end);
  }
  e.k_end = (int32_t)end;
  const int64_t lim = (int64_t)1 << 30;
  e.delta = (int32_t)(dl > lim ? lim : (dl < -lim ? -lim : dl));
  return e;
}

// Scalar description of one tile of BN keys, produced by the cursor.
struct TileInfo {
  uint32_t meta;            // run index | need-mask bit 16 | valid bit 17
  int32_t k0;               // first key of the tile inside its segment
  uint32_t so_k, so_v;      // byte offset of the tile's first row in the head's K / V
  uint32_t nrec_k, nrec_v;  // byte end of the segment in K / V (0 once exhausted)
  __device__ __forceinline__ bool valid() const { return (meta >> 17) & 1; }
  __device__ __forceinline__ bool need_mask() const { return (meta >> 16) & 1; }
  __device__ __forceinline__ int run() const { return meta & 0xffff; }
};

// Wave-uniform walk over the run table: tiles of BN keys in ring order.  A
// tile advance is a few scalar adds; the per-run values (byte ranges of the
// segment, the first key that needs a mask) are set up when a run starts.
struct RunCursor {
  int32_t ri, nruns, k0, k_end, thr;
  int32_t left;  // tiles still to produce (the workgroup's KV range)
  uint32_t so_k, so_v, nrec_k, nrec_v;
  bool done;
  __device__ __forceinline__ void load(const Run* runs, uint32_t kss, uint32_t vss, int32_t p0, bool causal) {
    const Run e = runs[ri];
    const int32_t kv_row = __builtin_amdgcn_readfirstlane(e.kv_row);
    const int32_t kv_len = __builtin_amdgcn_readfirstlane(e.kv_len);
    const int32_t delta = __builtin_amdgcn_readfirstlane(e.delta);
    k_end = __builtin_amdgcn_readfirstlane(e.k_end);
    // a tile starting at k0 crosses the segment end when k0 > kv_len - BN and
    // the diagonal of the wave's rows when k0 > delta + p0 - (BN - 1)
    const int32_t t_end = kv_len - BN;
    const int32_t t_diag = delta + p0 - (BN - 1);
    thr = (causal && t_diag < t_end) ? t_diag : t_end;
    so_k = (uint32_t)kv_row * kss;
    so_v = (uint32_t)kv_row * vss;
    nrec_k = (uint32_t)(kv_row + kv_len - 1) * kss + 2 * D;
    nrec_v = (uint32_t)(kv_row + kv_len - 1) * vss + 2 * D;
  }
  __device__ __forceinline__ void skip_empty(const Run* runs, uint32_t kss, uint32_t vss, int32_t p0, bool causal) {
    while (!done && k0 >= k_end) {
      if (++ri >= nruns) { done = true; nrec_k = nrec_v = 0; break; }
      k0 = 0;
      load(runs, kss, vss, p0, causal);
    }
  }
  // Start at tile `first` of the walk (whole runs are skipped by their tile
  // counts) and produce at most `count` tiles.
  __device__ __forceinline__ void start(const Run* runs, int32_t n, uint32_t kss, uint32_t vss, int32_t p0,
                                        bool causal, int32_t first, int32_t count) {
    nruns = n; ri = 0; k0 = 0; left = count; done = n <= 0 || count <= 0;
    k_end = thr = 0;
    so_k = so_v = nrec_k = nrec_v = 0;
    if (done) return;
    while (ri < nruns) {
      const int32_t nt = (__builtin_amdgcn_readfirstlane(runs[ri].k_end) + BN - 1) / BN;
      if (first < nt) break;
      first -= nt;
      ++ri;
    }
    if (ri >= nruns) { done = true; return; }
    load(runs, kss, vss, p0, causal);
    k0 = first * BN;
    so_k += (uint32_t)k0 * kss;
    so_v += (uint32_t)k0 * vss;
    skip_empty(runs, kss, vss, p0, causal);
  }
  __device__ __forceinline__ TileInfo tile() const {
    TileInfo t;
    t.meta = (uint32_t)ri | ((k0 > thr ? 1u : 0u) << 16) | ((done ? 0u : 1u) << 17);
    t.k0 = k0;
    t.so_k = so_k; t.so_v = so_v; t.nrec_k = nrec_k; t.nrec_v = nrec_v;
    return t;
  }
  __device__ __forceinline__ void advance(const Run* runs, uint32_t kss, uint32_t vss, int32_t p0, bool causal) {
    k0 += BN;
    so_k += BN * kss;
    so_v += BN * vss;
    if (--left <= 0) { done = true; nrec_k = nrec_v = 0; return; }
    skip_empty(runs, kss, vss, p0, causal);
  }
};

// EXACT: track the exact running maximum (chunk and step modes hand back the
// state relative to it); ring mode needs only the reference.
template <bool EXACT>
__global__ __launch_bounds__(NTHREADS, 1) void attn_fwd_bf16_kernel(FwdArgs a) {
  // four distinct arrays, so that the compiler can tell the buffer being
  // filled from the one being read and inserts no wait between them
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf0[KTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf1[KTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf0[VTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf1[VTILE];
  __shared__ Run runs[MAX_RUNS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;       // 0: group A, 1: group B
  const int l32 = lane & 31;
  const int g = lane >> 5;         // half-wave

  const WorkItem it = decode_work(a, blockIdx.x);
  const QGeom qg = query_geom(a, it);
  const int HP = a.heads_per_wg;
  const int G = a.hq / a.hkv;
  const int h = it.kvh * G + it.hg * HP + (wave % HP);
  const int wg_p0 = it.tile * a.rows_per_wg;
  const int p0 = __builtin_amdgcn_readfirstlane(wg_p0 + (wave / HP) * WAVE_ROWS);  // first row of this wave
  const int wg_p_hi = min(wg_p0 + a.rows_per_wg, qg.len) - 1;
  const int nruns = a.mode == MODE_CHUNK ? 1
                    : (a.mode == MODE_STEP ? 1 : a.n_chunks) * num_segments(a.layout);
  for (int r = tid; r < nruns; r += NTHREADS) runs[r] = make_run(a, qg, wg_p_hi, r);
  const int my_p = p0 + l32;                        // this lane's query row

  const __bf16* Qg = (const __bf16*)a.q + (int64_t)it.b * a.q_sb + (int64_t)h * a.q_sh;
  const unsigned char* Kg = (const unsigned char*)a.k + ((int64_t)it.b * a.k_sb + (int64_t)it.kvh * a.k_sh) * 2;
  const unsigned char* Vg = (const unsigned char*)a.v + ((int64_t)it.b * a.v_sb + (int64_t)it.kvh * a.v_sh) * 2;
  // row strides in bytes; every byte offset inside one head's K or V fits in
  // 31 bits (checked on the host)
  const uint32_t kss = (uint32_t)(a.k_ss * 2), vss = (uint32_t)(a.v_ss * 2);

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
  // chunk / step modes (EXACT): the incoming m (natural) and its base-2 image;
  // a row whose maximum does not move hands m back unchanged, not re-rounded
  float m_in = -INFINITY, m_in2 = -INFINITY;
  f32x16 acc[4];  // acc[dvb]: O^T[dv = dvb*32 + 8(r/4) + 4g + r%4][query my_p]
#pragma unroll
  for (int dvb = 0; dvb < 4; ++dvb) acc[dvb] = f32x16{};
  if (a.mode != MODE_RING && my_p < qg.len) {
    const int64_t mi = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + qg.row_base + my_p;
    const float mv = a.m[mi];
    m_ref = mv == -INFINITY ? -INFINITY : mv * LOG2E;
    m_max = m_ref;
    if constexpr (EXACT) {
      m_in = mv;
      m_in2 = m_ref;
    }
    l_run = g == 0 ? a.l[mi] : 0.f;
    const float* orow = a.o + (int64_t)it.b * a.o_sb + (int64_t)h * a.o_sh + (qg.row_base + my_p) * a.o_ss;
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

  // ---- staging: each group moves its half of every tile (keys 32 grp ..
  // 32 grp + 31) with buffer loads that write LDS directly (16 bytes per lane,
  // lane l to byte 16 l of a 1 KiB block).  Loads are relative to the tile's
  // KV segment; rows past the segment end are out of range and arrive as
  // zeros (masked keys must meet finite V), so no bounds branches are needed.
  const int wv = __builtin_amdgcn_readfirstlane(wave & 3);  // wave inside the group
  // K: wave wv fills row block 2 grp + wv / 2, chunks 8 (wv % 2) .. + 7
  const int k_rb = 2 * grp + (wv >> 1);
  int k_dst[2];
  uint32_t k_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = 2 * (wv & 1) + i;  // 1 KiB block inside the row block: chunks 4 blk .. 4 blk + 3
    k_dst[i] = __builtin_amdgcn_readfirstlane(k_rb * 4096 + blk * 1024);
    k_src[i] = (uint32_t)(16 * k_rb + (lane & 15)) * kss + (uint32_t)(4 * blk + (lane >> 4)) * 16;
  }
  // V: wave wv fills key rows 32 grp + 8 wv .. + 7, four rows per block; the
  // lane that lands on stored chunk lane % 16 of row r fetches chunk
  // (lane % 16) ^ 4 (r % 4), with r % 4 = lane / 16
  int v_dst[2];
  uint32_t v_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r0 = 32 * grp + 8 * wv + 4 * i;
    v_dst[i] = __builtin_amdgcn_readfirstlane(r0 * ROWB);
    v_src[i] = (uint32_t)(r0 + (lane >> 4)) * vss + (uint32_t)(((lane & 15) ^ ((lane >> 4) << 2)) << 4);
  }

  // Buffer resources span the head's whole K or V buffer up to the end of the
  // tile's segment: rows past the segment end read as zero, and an exhausted
  // cursor gets an empty range (its loads write zeros).
  // one 1 KiB block: j = 0, 1 K blocks of tile tk, j = 2, 3 V blocks of tile tv
  auto stage_block = [&](int j, const TileInfo& tk, unsigned char* kb, const TileInfo& tv, unsigned char* vb)
      __attribute__((always_inline)) {
    if (j < 2) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)Kg, (short)0, (int)tk.nrec_k, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(kb + k_dst[j]), 16, k_src[j], (int)tk.so_k, 0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)Vg, (short)0, (int)tv.nrec_v, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(vb + v_dst[j - 2]), 16, v_src[j - 2], (int)tv.so_v, 0, 0);
    }
  };

  // Per-lane LDS offsets of the MFMA operands inside one tile buffer; the
  // steps of a slot add compile-time constants.
  // K operand of (b2, ks): rows kperm(l32) + 32 b2, chunk 2 ks + g
  const int k_lane = k_pos(kperm(l32), g);  // + 8192 b2 + 512 ks
  // V^T operand of (dvb, b2, mm): dv = 32 dvb + l32, keys 32 b2 + 16 mm + 8 g
  // + 0..7, as two transposing reads of 4 keys.  In a read, lane 16 G + j
  // (j < 16) addresses key row (4 keys) + j / 4 at dv 32 dvb + 16 (G % 2) +
  // 4 (j % 4); the transpose hands lane 16 G + j the 4 keys of dv
  // 32 dvb + 16 (G % 2) + j.
  int v_lane[4];
  {
    const int G = lane >> 4, j = lane & 15, q = j >> 2;
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb)
      v_lane[dvb] = (8 * g + q) * ROWB + ((((dvb ^ q) << 2) + 2 * (G & 1) + ((j & 3) >> 1)) << 4) + (j & 1) * 8;
  }

  // Mask a tile: register r of block b2 in half-wave g is tile key
  // b2*32 + 16*(r/8) + 8g + r%8; it is hidden from this lane's row when key > lim.
  f32x16 s[2];       // S^T of a tile, between its matrix slot and its vector slot
  bf16x8 pf[2][2];   // P^T of a tile, between its vector slot and its PV MFMAs:
                     // pf[b2][mm] holds tile keys b2*32 + 16mm + 8g + 0..7
  // Masking (tiles that cross the diagonal or the segment end only): the
  // run's length and causal offset come from the run table.
  auto apply_mask = [&](const TileInfo& t) __attribute__((always_inline)) {
    const Run e = runs[t.run()];
    const int kv_len = __builtin_amdgcn_readfirstlane(e.kv_len);
    const int delta = __builtin_amdgcn_readfirstlane(e.delta);
    int lim = kv_len - 1 - t.k0;
    if (causal) {
      const int lc = my_p + delta - t.k0;
      lim = lc < lim ? lc : lim;
    }
    const int lim32 = (lim < -1 ? -1 : (lim > 1000 ? 1000 : lim)) - 8 * g;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = b2 * 32 + 16 * (r >> 3) + (r & 7);
        s[b2][r] = kk > lim32 ? -INFINITY : s[b2][r];
      }
  };

  // Exponentials of a computed S^T against the reference m_use into P^T, and
  // this lane's part of the tile's row sum (fp32 adds in four chains; not
  // v_dot2 over the bf16 pairs: dot instructions wait for the matrix core,
  // which the other wave of the SIMD keeps busy during this slot).
  auto exponentials = [&](float m_use, auto side) __attribute__((always_inline)) -> float {
    float rs[4];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[b2][mm * 8 + e], c2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[b2][mm * 8 + e + 1], c2, -m_use));
          pf[b2][mm][e] = (__bf16)p0;
          pf[b2][mm][e + 1] = (__bf16)p1;
          float& r = rs[2 * b2 + mm];
          r = e == 0 ? p0 + p1 : (r + p0) + p1;
          if (b2 == 0 && mm == 1 && e == 6) side(2);
        }
    return (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };
  // Tile maximum (two chains of three-input maxima over the lane's 32 scores,
  // then the other half-wave), in log2 units.
  auto tile_max = [&]() __attribute__((always_inline)) -> float {
    float mx0 = fmaxf(s[0][0], s[0][1]), mx1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      mx0 = fmaxf(fmaxf(mx0, s[0][r]), s[0][r + 1]);
      mx1 = fmaxf(fmaxf(mx1, s[1][r]), s[1][r + 1]);
    }
    return max_pair32(fmaxf(mx0, mx1)) * c2;
  };
  // Move the reference of the lanes where `grow` holds to mx (rescaling O^T
  // and l); a no-op unless some lane grows.
  auto move_reference = [&](bool grow, float mx) __attribute__((always_inline)) {
    if (__any(grow)) {
      const float m_new = grow ? mx : m_ref;
      const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dvb = 0; dvb < 4; ++dvb) acc[dvb] *= alpha;
    }
  };

  // Vector work on a computed S^T: mask, reference update (rare O^T rescale),
  // exponentials into P^T and the row sum.  side(j), j = 0..3, is called at
  // four points spread over the work.
  //   EXACT: the tile maximum first, as the pages' update does, tracking the
  //     exact running maximum beside the reference (the state handed back by
  //     the chunk entry point is relative to it); the reference moves when
  //     the maximum exceeds it by more than RESCALE_SLACK.
  //   otherwise: the exponentials first, against the current reference.  A
  //     lane whose 32 values sum to at most 2^8 has every P^T value at most
  //     2^8, the same bound the lazy reference keeps; if any lane's sum is
  //     larger or not finite (as while the reference is still -inf) the tile maximum
  //     is taken, the reference moves to it wherever it grew, and the
  //     exponentials are recomputed.  The result is the same update with the
  //     maximum skipped on nearly every tile.
  auto softmax_tile = [&](const TileInfo& t, auto side) __attribute__((always_inline)) {
    side(0);
    if (t.need_mask()) apply_mask(t);
    auto nothing = [](int) {};
    if constexpr (EXACT) {
      const float mx = tile_max();
      m_max = fmaxf(m_max, mx);
      move_reference(mx > m_ref + RESCALE_SLACK, mx);  // also true when m_ref is -inf
      side(1);
      l_run += exponentials(m_ref == -INFINITY ? 0.f : m_ref, side);
    } else {
      side(1);
      float part = exponentials(m_ref, side);
      // part is a sum of exponentials, so not negative: as an unsigned bit
      // pattern it exceeds that of 2^8 exactly when it is larger than 2^8,
      // infinite (as while the reference is still -inf) or NaN; one compare
      // instead of two and the merge of their masks
      if (__builtin_amdgcn_ballot_w64(__float_as_uint(part) > 0x43800000u) != 0) {
        const float mx = tile_max();
        move_reference(mx > m_ref, mx);
        part = exponentials(m_ref == -INFINITY ? 0.f : m_ref, nothing);
      }
      l_run += part;
    }
    side(3);
  };

  // MFMA operand reads from the K buffer KB / V buffer VB of a slot, step i
  // (i = 0..15: QK half b2 = i % 2 at 16-key step i / 2, PV 16-key step
  // i / 4 at dv block i % 4)
  auto kread = [&](auto kbc, int i) __attribute__((always_inline)) {
    const unsigned char* kb = decltype(kbc)::value ? kbuf1 : kbuf0;
    return *(const bf16x8*)(kb + k_lane + (i & 1) * 8192 + (i >> 1) * 512);
  };
  auto vread = [&](auto vbc, int i) __attribute__((always_inline)) {
    const unsigned char* vb = decltype(vbc)::value ? vbuf1 : vbuf0;
    const int pb2 = i >> 3, pmm = (i >> 2) & 1, dvb = i & 3;
    const unsigned char* p = vb + v_lane[dvb] + (32 * pb2 + 16 * pmm) * ROWB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * ROWB));
    const s16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
  };
  constexpr int AHEAD = 2;  // operand reads in flight per chain
  bf16x8 kq[AHEAD], vq[AHEAD];
  auto first_reads = [&](auto kbc, auto vbc) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
      kq[i] = kread(kbc, i);
      vq[i] = vread(vbc, i);
    }
  };

  // Matrix slot: S^T of the tile in K buffer KB and O^T += V^T P^T with the
  // tile in V buffer VB; the two MFMA chains alternate so that each operand
  // read has time to land.  At the ends of the stream one half works on stale
  // or zero data: a QK with no tile behind it is never used, and the first PV
  // multiplies P^T = 0 with a zeroed V buffer.  With `pre` the first reads
  // were issued before the slot began.
  auto matrix_slot = [&](auto kbc, auto vbc, auto side, auto pre) __attribute__((always_inline)) {
    if constexpr (!decltype(pre)::value) {
      first_reads(kbc, vbc);
      __builtin_amdgcn_sched_barrier(0);  // the first reads go out before anything else
    }
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8 kf = kq[i % AHEAD], vf = vq[i % AHEAD];
      if (i + AHEAD < 16) {
        kq[i % AHEAD] = kread(kbc, i + AHEAD);
        vq[i % AHEAD] = vread(vbc, i + AHEAD);
      }
      // keep the reads issued ahead of the two MFMAs that follow
      __builtin_amdgcn_sched_barrier(0);
      const int ks = i >> 1, b2 = i & 1;
      s[b2] = mfma(kf, qf[ks], s[b2]);
      const int pb2 = i >> 3, pmm = (i >> 2) & 1, dvb = i & 3;
      acc[dvb] = mfma(vf, pf[pb2][pmm], acc[dvb]);
      __builtin_amdgcn_sched_barrier(0);
      side(i);  // staging issue placed between MFMA pairs
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- tile stream: infos of tiles n-1 .. n+2 around loop iteration n
  __syncthreads();  // run table complete
  RunCursor cur;
  {
    const int32_t nr = wg_p_hi < wg_p0 ? 0 : nruns;
    int32_t first = 0, count = 0x7fffffff;
    if (a.kv_splits > 1) {
      // this workgroup's range of the walk: tiles [T s / S, T (s + 1) / S)
      int64_t total = 0;
      for (int r = 0; r < nr; ++r) total += (__builtin_amdgcn_readfirstlane(runs[r].k_end) + BN - 1) / BN;
      const int64_t tb = total * it.split / a.kv_splits, te = total * (it.split + 1) / a.kv_splits;
      first = (int32_t)tb;
      count = (int32_t)(te - tb);
    }
    cur.start(runs, nr, kss, vss, p0, causal, first, count);
  }
  auto next_info = [&]() __attribute__((always_inline)) -> TileInfo {
    const TileInfo t = cur.tile();
    if (!cur.done) cur.advance(runs, kss, vss, p0, causal);
    return t;
  };
  // ring of tile infos: around loop iteration n, ti[n % 4] is tile n and
  // ti[(n + 3) % 4] tile n - 1 (the slot of tile n + 3 once it is produced)
  TileInfo ti[4];
  ti[3].meta = 0;  // tile -1: invalid
  ti[3].k0 = 0;
  ti[3].so_k = ti[3].so_v = ti[3].nrec_k = ti[3].nrec_v = 0;
  ti[0] = next_info();
  ti[1] = next_info();
  ti[2] = next_info();

  // prologue: K(0) into K buffer 0 (both groups, one half each), both V
  // buffers zeroed (the first PV multiplies P^T = 0 with V buffer 1, and every
  // later V byte is finite tile data), P^T zeroed, S^T = -inf (tile -1)
  stage_block(0, ti[0], kbuf0, ti[0], vbuf0);
  stage_block(1, ti[0], kbuf0, ti[0], vbuf0);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    *(u32x4*)(vbuf0 + tid * 32 + 16 * c) = u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)(vbuf1 + tid * 32 + 16 * c) = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) {
    s[b2] = f32x16{} - INFINITY;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) pf[b2][mm] = bf16x8{};
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K(0) is in LDS
  __syncthreads();

  // Barrier at the end of an iteration.  Not __syncthreads(): its release
  // fence would also wait for LDS reads in flight; the staging loads are
  // waited for explicitly just before it.  No buffer read in an iteration is
  // written before the next one, so a barrier between the two slots is not
  // needed (and measured 0.9 % slower).
  auto slot_barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Loop iteration n (two slots, a barrier after the second):
  //   slot 1: A matrix (QK(n), PV(n-1))  |  B vector (softmax(n-1))
  //   slot 2: A vector (softmax(n))  |  B matrix (QK(n), PV(n-1))
  // Staging of K(n+1) into K buffer (n+1) % 2 and of V(n) into V buffer n % 2
  // is issued in slot 1 by both groups, one 1 KiB block per wave at a time
  // (group A after every other MFMA pair of the second half of its matrix
  // slot, group B spread over its softmax),
  // and waited for at the end of slot 2; neither buffer is read in iteration n.
  auto iteration = [&](auto qc) __attribute__((always_inline)) {
    constexpr int Q = decltype(qc)::value;   // n % 4
    constexpr int P = Q & 1;                 // n % 2
    const std::integral_constant<int, P> kbc{};
    const std::integral_constant<int, P ^ 1> vbc{};
    const TileInfo& tm1 = ti[(Q + 3) & 3];
    const TileInfo& t0 = ti[Q];
    const TileInfo& t1 = ti[(Q + 1) & 3];
    auto stage = [&](int j) __attribute__((always_inline)) {
      stage_block(j, t1, P ? kbuf0 : kbuf1, t0, P ? vbuf1 : vbuf0);
    };
    auto stage_late = [&](int i) __attribute__((always_inline)) {
      if (i >= 8 && (i & 1) == 0) stage((i - 8) >> 1);
    };
    auto nothing = [&](int) __attribute__((always_inline)) {};
    const std::false_type read_first{};
    const std::true_type prefetched{};
    if (grp == 0) {
      matrix_slot(kbc, vbc, stage_late, read_first);
    } else {
      // also on tile -1 (iteration 0), where S^T = -inf makes it a no-op
      // that leaves P^T = 0: the staging blocks are issued from inside it
      softmax_tile(tm1, stage);
      // the first operands of this group's matrix slot: K(n) and V(n-1) are
      // complete since the previous iteration
      first_reads(kbc, vbc);
    }
    if (grp == 0) {
      if (t0.valid()) softmax_tile(t0, nothing);
    } else {
      matrix_slot(kbc, vbc, nothing, prefetched);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's staging has landed
    slot_barrier();
    ti[(Q + 3) & 3] = next_info();  // tile n + 3 takes the place of tile n - 1
  };
  for (;;) {
    if (!(ti[0].valid() || ti[3].valid())) break;
    iteration(std::integral_constant<int, 0>{});
    if (!(ti[1].valid() || ti[0].valid())) break;
    iteration(std::integral_constant<int, 1>{});
    if (!(ti[2].valid() || ti[1].valid())) break;
    iteration(std::integral_constant<int, 2>{});
    if (!(ti[3].valid() || ti[2].valid())) break;
    iteration(std::integral_constant<int, 3>{});
  }

  // ---- epilogue
  float lt = sum_pair32(l_run);
  if (my_p >= qg.len) return;
  if (a.mode == MODE_RING && a.kv_splits > 1) {
    // partial of this KV range: normalized o and natural lse
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t prow = (((int64_t)it.split * a.batch + it.b) * a.hq + h) * a.part_rows + qg.row_base + my_p;
    float* orow = a.part_o + prow * D;
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[dvb][r4 * 4 + e] * inv;
        *(f32x4*)(orow + dvb * 32 + r4 * 8 + 4 * g) = v4;
      }
    if (g == 0) a.part_lse[prow] = lt > 0.f ? (m_ref + __log2f(lt)) * LN2 : -INFINITY;
  } else if (a.mode == MODE_RING) {
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
    // chunk / step mode: hand back the state relative to the exact running maximum
    const float f = (m_max == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_max);
    lt *= f;
    const int64_t mi = (int64_t)it.b * a.ml_sb + (int64_t)h * a.ml_sh + qg.row_base + my_p;
    if (g == 0) {
      if constexpr (EXACT) a.m[mi] = m_max == m_in2 ? m_in : m_max * LN2;
      else a.m[mi] = m_max == -INFINITY ? -INFINITY : m_max * LN2;
      a.l[mi] = lt;
    }
    float* orow = a.o + (int64_t)it.b * a.o_sb + (int64_t)h * a.o_sh + (qg.row_base + my_p) * a.o_ss;
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
  if (a.mode != MODE_RING)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<true>, dim3(a.n_work), dim3(NTHREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<false>, dim3(a.n_work), dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ra
