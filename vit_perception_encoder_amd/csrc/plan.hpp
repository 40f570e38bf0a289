// Work split of one mgattn_dense call: segments -> launches -> workgroups.
//
// Host side: the caller's cu_seqlens (a host array) is validated, empty segments are
// dropped, the rest are ordered longest first and packed into launches of at most
// kMaxSegPerLaunch segments.  Each launch carries its segment table by value in the
// kernel arguments, so no device memory is allocated and no device->host sync is
// needed.  Windows and whole images are both just segments, so window and full
// layers share one launch shape: vllm.cpp issue #1545, section "The fix" (the
// block-diagonal mask is per-segment row slices).
//
// Device side: decode_tile() maps a workgroup id to (segment slot, head, first query
// of its q-tile).  When H is a multiple of 8, heads are dealt to the eight XCDs
// (workgroup b runs on XCD b % 8), so the q-tiles of one (segment, head) share one
// L2 and every XCD gets the same mix of long and short segments.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <limits>
#include <vector>

namespace mgattn {

constexpr int kMaxSegPerLaunch = 120;
constexpr int kXcds = 8;

// Segment table of one launch (plain data, copied into the kernel arguments).
struct SegTable {
  int32_t n;                                // segments in this launch
  int32_t nx;                               // XCD groups: 8 if H % 8 == 0, else 1
  int32_t start[kMaxSegPerLaunch];          // first query token of each segment
  int32_t len[kMaxSegPerLaunch];            // queries in each segment (> 0)
  int32_t kstart[kMaxSegPerLaunch];         // first key token (= start without a KV cache)
  int32_t klen[kMaxSegPerLaunch];           // keys (>= len; = len without a KV cache)
  int32_t tile_prefix[kMaxSegPerLaunch + 1];  // exclusive prefix of ceil(len * rows_per_token / block_m)
};

struct Tile {
  int32_t slot;   // index into SegTable
  int32_t head;
  int32_t q0;     // first query of the q-tile, relative to the segment start
  int32_t valid;  // 0 for an idle workgroup id
};

// Workgroup id -> tile.  Within an XCD group the order is: segments longest first,
// then heads, then q-tiles (causal: last q-tile first, as it sees the most keys).
__host__ __device__ inline Tile decode_tile(const SegTable& t, int H, int block_m, int causal, int b) {
  Tile r = {0, 0, 0, 0};
  const int nx = t.nx;
  const int x = b % nx;
  const int i = b / nx;
  const int hx = H / nx;
  if (i >= t.tile_prefix[t.n] * hx) return r;
  int lo = 0, hi = t.n;  // tile_prefix[lo]*hx <= i < tile_prefix[hi]*hx
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (t.tile_prefix[mid] * hx <= i) lo = mid; else hi = mid;
  }
  const int nq = t.tile_prefix[lo + 1] - t.tile_prefix[lo];
  const int local = i - t.tile_prefix[lo] * hx;
  const int hh = local / nq;
  int qt = local - hh * nq;
  if (causal) qt = nq - 1 - qt;
  r.slot = lo;
  r.head = x + nx * hh;
  r.q0 = qt * block_m;
  r.valid = 1;
  return r;
}

// One launch of the plan: its table and, for introspection, each slot's index in the
// caller's cu_seqlens.
struct Launch {
  SegTable table;
  std::vector<int> orig;
  int64_t grid;
};

// Builds the launches for already-validated arguments.  cuk (may be NULL: keys are
// the queries) gives each segment's key rows when queries attend a longer key range
// (a KV cache).  Returns false if a launch would need more workgroups than a grid
// dimension holds.
// rows_per_token: query rows of a token in one tile (the query heads packed per
// key/value head; 1 when every query head has its own tiles).
inline bool make_plan(const int32_t* cu, const int32_t* cuk, int n_seg, int H, int block_m,
                      std::vector<Launch>& out, int rows_per_token = 1) {
  struct Seg { int32_t start, len, kstart, klen; int orig; };
  std::vector<Seg> segs;
  segs.reserve(n_seg);
  for (int g = 0; g < n_seg; ++g) {
    const int32_t len = cu[g + 1] - cu[g];
    const int32_t ks = cuk ? cuk[g] : cu[g];
    const int32_t kl = cuk ? cuk[g + 1] - cuk[g] : len;
    if (len > 0) segs.push_back({cu[g], len, ks, kl, g});
  }
  std::stable_sort(segs.begin(), segs.end(), [](const Seg& a, const Seg& b) { return a.len > b.len; });
  out.clear();
  const int nx = (H % kXcds == 0) ? kXcds : 1;
  for (size_t s0 = 0; s0 < segs.size(); s0 += kMaxSegPerLaunch) {
    const size_t n = std::min<size_t>(kMaxSegPerLaunch, segs.size() - s0);
    Launch l;
    l.table = SegTable{};
    l.table.n = static_cast<int32_t>(n);
    l.table.nx = nx;
    int64_t tiles = 0;
    l.table.tile_prefix[0] = 0;
    for (size_t j = 0; j < n; ++j) {
      const Seg& s = segs[s0 + j];
      l.table.start[j] = s.start;
      l.table.len[j] = s.len;
      l.table.kstart[j] = s.kstart;
      l.table.klen[j] = s.klen;
      tiles += (static_cast<int64_t>(s.len) * rows_per_token + block_m - 1) / block_m;
      if (tiles * H > std::numeric_limits<int32_t>::max()) return false;
      l.table.tile_prefix[j + 1] = static_cast<int32_t>(tiles);
      l.orig.push_back(s.orig);
    }
    l.grid = tiles * H;
    out.push_back(std::move(l));
  }
  return true;
}

}  // namespace mgattn
