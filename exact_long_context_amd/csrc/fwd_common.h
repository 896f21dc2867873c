// Work decomposition and the KV-tile cursor shared by the forward kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"
#include "schedule.h"

namespace ra {

// What one workgroup computes: one query segment tile of `rows_per_wg` rows
// for `heads_per_wg` query heads that share one KV head.
struct WorkItem {
  int32_t b, kvh, hg;      // batch, KV head, query-head group inside the KV head
  int32_t qc_idx;          // query chunk index relative to q_first (ring) / 0 (chunk)
  int32_t qsi;             // query segment index inside the chunk
  int32_t tile;            // tile index along the segment
  int32_t split;           // KV range (0 .. kv_splits - 1)
};

// Workgroups are numbered heaviest-first (causal work grows with the token
// position of the rows), and, when the KV streams split evenly over the 8
// XCDs, workgroup w lands on XCD w % 8 together with the other workgroups of
// the same KV stream, so that tiles walking the same keys share that XCD's L2.
// With xcd_swizzle = S in {2, 4} the streams are taken S at a time over the
// whole chip instead (XCD w % 8 serves stream w % S of the current group),
// one group after another: the K / V of the streams in flight then stays
// within the memory-side cache, where walking all streams at once would not.
// With xcd_swizzle = 3 (streams that do not split over the XCDs, a multiple of
// 256 workgroups) XCD w % 8 takes blocks of 32 consecutive workgroups of the
// heaviest-first order, block b on XCD b % 8: the 32 workgroups an XCD runs at
// a time are neighbouring tiles that walk the same keys in step, and the
// blocks of every weight spread over all XCDs.
// The KV ranges of one query tile (split-KV) take consecutive ranks.
__device__ __forceinline__ WorkItem decode_work(const FwdArgs& a, int32_t w) {
  const int32_t G = a.hq / a.hkv;
  const int32_t hg_count = G / a.heads_per_wg;
  const int32_t n_streams = a.batch * a.hkv;
  int32_t r, stream, hg;
  if (a.xcd_swizzle == 3) {
    const int32_t x = w & 7, u = w >> 3;
    w = (((u >> 5) << 3) + x) * 32 + (u & 31);
  }
  if (a.xcd_swizzle == 2 || a.xcd_swizzle == 4) {
    const int32_t S = a.xcd_swizzle;
    const int32_t per_s = a.n_work / n_streams;  // workgroups per stream
    const int32_t grp = w / (S * per_s);
    const int32_t rem = w - grp * S * per_s;
    stream = S * grp + rem % S;
    const int32_t v = rem / S;
    r = v / hg_count;
    hg = v - r * hg_count;
  } else if (a.xcd_swizzle == 1) {
    const int32_t x = w & 7, u = w >> 3;
    const int32_t per = (n_streams >> 3) * hg_count;
    r = u / per;
    const int32_t rem = u - r * per;
    stream = x + 8 * (rem / hg_count);
    hg = rem % hg_count;
  } else {
    const int32_t per = n_streams * hg_count;
    r = w / per;
    const int32_t rem = w - r * per;
    stream = rem / hg_count;
    hg = rem % hg_count;
  }
  WorkItem it;
  it.split = r % a.kv_splits;
  r /= a.kv_splits;
  it.b = stream / a.hkv;
  it.kvh = stream % a.hkv;
  it.hg = hg;
  const int32_t tps = a.tiles_per_seg;
  it.qsi = 0;
  if (a.mode == MODE_CHUNK) {
    it.qc_idx = 0;
    it.tile = tps - 1 - r;
  } else if (a.layout == ZIGZAG) {
    // late segments first (every late token is later than every early one),
    // later tokens first inside a segment
    const int32_t sr = r / tps;
    it.tile = tps - 1 - (r - sr * tps);
    if (sr < a.q_count) { it.qc_idx = sr; it.qsi = 1; }
    else { it.qc_idx = a.q_count - 1 - (sr - a.q_count); it.qsi = 0; }
  } else if (a.layout == STRIPED) {
    const int32_t tr = r / a.q_count;
    it.tile = tps - 1 - tr;
    it.qc_idx = a.q_count - 1 - (r - tr * a.q_count);
  } else {
    const int32_t cr = r / tps;
    it.qc_idx = a.q_count - 1 - cr;
    it.tile = tps - 1 - (r - cr * tps);
  }
  return it;
}

// Query-side geometry of a work item.
struct QGeom {
  Segment seg;        // query segment (positions)
  int32_t len;        // rows in the segment
  int64_t row_base;   // buffer row of the segment's row 0 (q / out / lse / state)
  int32_t qchunk;     // global query chunk index (ring)
};

__device__ __forceinline__ QGeom query_geom(const FwdArgs& a, const WorkItem& it) {
  QGeom g;
  if (a.mode == MODE_CHUNK) {
    g.seg.row0 = 0; g.seg.len = a.lq; g.seg.base = 0; g.seg.step = 1;
    g.len = a.lq;
    g.row_base = 0;
    g.qchunk = 0;
  } else {
    const int32_t L = a.lq;  // chunk length
    g.qchunk = a.q_first + it.qc_idx;
    g.seg = segment_l(a.layout, L, a.n_chunks, g.qchunk, it.qsi);
    g.len = g.seg.len;
    g.row_base = (int64_t)it.qc_idx * L + g.seg.row0;
  }
  return g;
}

// Walks the KV tiles a workgroup must visit, in ring order: step t visits KV
// chunk (q - t) mod N, its segments in row order, keys ascending inside a
// segment (step mode: only step a.step, in a buffer holding that chunk).
// Tiles wholly in the future of the workgroup's last row are never produced;
// segment pairs classified SKIP produce no tile at all.
template <int BN>
struct TileCursor {
  // fixed
  int32_t mode, layout, n, causal, nseg, L;
  int64_t seq;
  int32_t qchunk;
  Segment qseg;
  int32_t p_hi;          // last valid query row of the workgroup in the segment
  int32_t lk;            // chunk mode: key rows
  int64_t delta_chunk;   // chunk mode: causal offset
  int32_t t_first, t_end;  // ring steps walked
  // moving
  int32_t t, sb;         // ring step, KV segment index
  int32_t k0;            // first key of the tile, relative to the segment
  int64_t kv_row;        // buffer row of the KV segment's row 0
  int32_t kv_len;        // rows in the KV segment
  int32_t k_end;         // keys to visit in this segment
  int32_t delta;         // causal offset, clamped to [-(2^30), 2^30]
  bool done;

  __device__ __forceinline__ void load_run() {
    int64_t dl = 0;
    if (mode == MODE_CHUNK) {
      kv_row = 0;
      kv_len = lk;
      dl = delta_chunk;
    } else {
      const int32_t j = ring_kv_chunk(qchunk, t, n);
      const Segment ks = segment_l(layout, L, n, j, sb);
      kv_row = (mode == MODE_STEP ? 0 : (int64_t)j * L) + ks.row0;
      kv_len = ks.len;
      dl = causal ? pair_delta(qseg, ks) : 0;
    }
    int64_t end = kv_len;
    if (causal) {
      const int64_t e = (int64_t)p_hi + dl + 1;
      end = e < 0 ? 0 : (e < end ? e : end);
    }
    k_end = (int32_t)end;
    const int64_t lim = (int64_t)1 << 30;
    delta = (int32_t)(dl > lim ? lim : (dl < -lim ? -lim : dl));
  }

  __device__ __forceinline__ void skip_empty() {
    while (!done && k0 >= k_end) {
      if (++sb >= nseg) { sb = 0; ++t; }
      if (t >= t_end) { done = true; break; }
      k0 = 0;
      load_run();
    }
  }

  __device__ __forceinline__ void start() {
    t = t_first; sb = 0; k0 = 0; done = false;
    load_run();
    skip_empty();
  }

  __device__ __forceinline__ void advance() {
    k0 += BN;
    skip_empty();
  }
};

template <int BN>
__device__ __forceinline__ TileCursor<BN> make_cursor(const FwdArgs& a, const QGeom& qg, int32_t p_hi) {
  TileCursor<BN> c;
  c.mode = a.mode;
  c.layout = a.layout;
  c.n = a.n_chunks;
  c.causal = a.causal;
  c.nseg = a.mode == MODE_CHUNK ? 1 : num_segments(a.layout);
  c.L = a.mode == MODE_CHUNK ? a.lk : a.lq;
  c.seq = a.seq;
  c.qchunk = qg.qchunk;
  c.qseg = qg.seg;
  c.p_hi = p_hi;
  c.lk = a.lk;
  c.delta_chunk = a.delta;
  c.t_first = a.mode == MODE_STEP ? a.step : 0;
  c.t_end = a.mode == MODE_CHUNK ? 1 : (a.mode == MODE_STEP ? a.step + 1 : a.n_chunks);
  c.start();
  return c;
}

}  // namespace ra
