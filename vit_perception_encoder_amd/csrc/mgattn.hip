// C ABI of the mgattn library: argument checks, the launch plan and the launches.
//
// Conventions from the pages: the supported domain and the on-chip memory a launch
// requests are host arithmetic that needs no GPU, bounds are inclusive, and
// anything unsupported is refused by name before launching (vllm.cpp PR #1578,
// section "AttentionDenseFlash advertises the head_dim it can launch"); segment
// boundaries are checked before any slicing or launch (the vision-tower commit of
// vllm.cpp PR #279, where a coverage check placed after the slicing loop let a
// mutant hang).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/mgattn.h"
#include "attn_bf16.hpp"
#include "attn_bf16_pipe.hpp"
#include "attn_decode.hpp"
#include "attn_f32.hpp"
#include "plan.hpp"
#include "window_rope.hpp"

using namespace mgattn;

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool head_dim_ok(int d) { return d == 64 || d == 96 || d == 128; }
bool dtype_ok(int dt) { return dt == MGATTN_F32 || dt == MGATTN_BF16; }
size_t elem_size(int dt) { return dt == MGATTN_F32 ? 4 : 2; }

int block_m_of(int d, int dtype) {
  (void)d;
  return dtype == MGATTN_BF16 ? Bf16Tile<96>::kBlockM : F32Tile<96>::kBlockM;
}

// Workgroup shape of one dense call of the bf16 head_dim-96 kernel, which runs 8 or 4
// waves of 32 queries: 256 queries (8 waves) when the (segment, head, tile) units give
// at least one workgroup per CU.  With fewer, a non-causal call splits every tile's
// keys between wave groups (attn_fwd_bf16_pipe<.., G>): 128-query tiles of 8 waves in
// two groups when those fill the CUs, else 64-query tiles of 8 waves in four groups,
// each taking 32 keys of every 128 (a single 1024-token segment of 16 heads: 64 units
// of 256, 256 units of 64, two waves per SIMD, 8 steps of 32 keys per wave).  A causal
// call keeps whole keys per wave: 128-query tiles of 4 waves.  Other kernels have one
// tile height.
constexpr int kFillWorkgroups = 256;  // CUs of an MI355X
enum class DenseKind { kFull8, kFull4, kSplit8, kQuad8, kF32Split, kF32Split16, kOther };
int64_t dense_units(const int32_t* cu, int n_seg, int H, int bm) {
  int64_t units = 0;
  for (int g = 0; g < n_seg; ++g) units += (static_cast<int64_t>(cu[g + 1] - cu[g]) + bm - 1) / bm;
  return units * H;
}
DenseKind dense_kind(const int32_t* cu, int n_seg, int H, int d, int dtype, int causal) {
  // f32: 32-query blocks with the keys split over the workgroup's waves when the
  // 128-query tiles leave CUs idle (non-causal), 16-query blocks when those do too
  if (dtype == MGATTN_F32) {
    if (causal || dense_units(cu, n_seg, H, F32Tile<96>::kBlockM) >= kFillWorkgroups) return DenseKind::kOther;
    return dense_units(cu, n_seg, H, 32) >= kFillWorkgroups ? DenseKind::kF32Split : DenseKind::kF32Split16;
  }
  if (dtype != MGATTN_BF16 || d != 96) return DenseKind::kOther;
  if (dense_units(cu, n_seg, H, 256) >= kFillWorkgroups) return DenseKind::kFull8;
  if (causal) return DenseKind::kFull4;
  return dense_units(cu, n_seg, H, 128) >= kFillWorkgroups ? DenseKind::kSplit8 : DenseKind::kQuad8;
}
int dense_block_m(const int32_t* cu, int n_seg, int H, int d, int dtype, int causal) {
  switch (dense_kind(cu, n_seg, H, d, dtype, causal)) {
    case DenseKind::kFull8: return 256;
    case DenseKind::kFull4: return 128;
    case DenseKind::kSplit8: return 128;
    case DenseKind::kQuad8: return 64;
    case DenseKind::kF32Split: return 32;
    case DenseKind::kF32Split16: return 16;
    default: return block_m_of(d, dtype);
  }
}

long lds_bytes_of(int d, int dtype) {
  if (dtype == MGATTN_BF16) {
    switch (d) {
      case 64: return Bf16Tile<64>::kLdsBytes;
      case 96: return sched::pipe_lds_elems<96>(256) * 2;  // the pipelined kernel, 256-query tiles
      case 128: return Bf16Tile<128>::kLdsBytes;
    }
  } else {  // the largest of the three f32 workgroup shapes
    switch (d) {
      case 64: return std::max({F32Tile<64>::kLdsBytes + 0L, f32_split_lds_bytes<64>(), f32_split16_lds_bytes<64>()});
      case 96: return std::max({F32Tile<96>::kLdsBytes + 0L, f32_split_lds_bytes<96>(), f32_split16_lds_bytes<96>()});
      case 128:
        return std::max({F32Tile<128>::kLdsBytes + 0L, f32_split_lds_bytes<128>(), f32_split16_lds_bytes<128>()});
    }
  }
  return MGATTN_ERR_HEAD_DIM;
}

static_assert(Bf16Tile<64>::kBlockM == Bf16Tile<128>::kBlockM, "block_m must not depend on d");
static_assert(F32Tile<64>::kBlockM == F32Tile<128>::kBlockM, "block_m must not depend on d");

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Byte span of a [T rows of H*d elements, leading dimension ld] tensor.
size_t span_bytes(int64_t T, int64_t ld, int H, int d, int dtype) {
  return (static_cast<size_t>(T - 1) * static_cast<size_t>(ld) + static_cast<size_t>(H) * d) * elem_size(dtype);
}

// Prefix-sum array of n+1 entries: starts at 0, non-decreasing, total > 0.  Writes the
// total and the longest entry.
int check_seqlens(const int32_t* cu, int n, int64_t* total, int64_t* longest) {
  if (cu[0] != 0) return MGATTN_ERR_SEQLENS;
  int64_t m = 0;
  for (int g = 0; g < n; ++g) {
    if (cu[g + 1] < cu[g]) return MGATTN_ERR_SEQLENS;
    m = std::max<int64_t>(m, static_cast<int64_t>(cu[g + 1]) - cu[g]);
  }
  if (cu[n] <= 0) return MGATTN_ERR_SEQLENS;
  *total = cu[n];
  *longest = m;
  return MGATTN_OK;
}

// Checks every argument that needs no GPU.  ld* are the leading dimensions
// (elements between consecutive tokens).  Keys and values have Hkv heads and, when
// cuk is not NULL, their own segments (cuk[g+1] - cuk[g] >= cu[g+1] - cu[g]).
int validate(const void* q, const void* k, const void* v, void* out, int64_t ldq, int64_t ldk, int64_t ldv,
             int64_t ldo, const int32_t* cu, const int32_t* cuk, int n_seg, int H, int Hkv, int d, float scale,
             int causal, int window, int dtype) {
  if (!dtype_ok(dtype)) return MGATTN_ERR_DTYPE;
  if (!q || !k || !v || !out || !cu) return MGATTN_ERR_NULL;
  if (n_seg < 1) return MGATTN_ERR_SEGMENTS;
  if (H < 1 || Hkv < 1 || H % Hkv != 0) return MGATTN_ERR_HEADS;
  if (!head_dim_ok(d)) return MGATTN_ERR_HEAD_DIM;
  if (!isfinite(scale) || (causal != 0 && causal != 1)) return MGATTN_ERR_SCALE;
  if (window < 0) return MGATTN_ERR_WINDOW;
  const int64_t row_q = static_cast<int64_t>(H) * d, row_kv = static_cast<int64_t>(Hkv) * d;
  const int64_t align_elems = 16 / static_cast<int64_t>(elem_size(dtype));
  for (int64_t ld : {ldq, ldo})
    if (ld < row_q || ld > INT32_MAX || ld % align_elems != 0) return MGATTN_ERR_STRIDE;
  for (int64_t ld : {ldk, ldv})
    if (ld < row_kv || ld > INT32_MAX || ld % align_elems != 0) return MGATTN_ERR_STRIDE;
  int64_t Tq = 0, Tk = 0, max_q = 0, max_k = 0;
  int st = check_seqlens(cu, n_seg, &Tq, &max_q);
  if (st != MGATTN_OK) return st;
  if (cuk) {
    st = check_seqlens(cuk, n_seg, &Tk, &max_k);
    if (st != MGATTN_OK) return st;
    for (int g = 0; g < n_seg; ++g)
      if (cuk[g + 1] - cuk[g] < cu[g + 1] - cu[g]) return MGATTN_ERR_SEQLENS;
  } else {
    Tk = Tq;
    max_k = max_q;
  }
  if (max_q * (H / Hkv) > INT32_MAX) return MGATTN_ERR_SIZE;  // packed query rows of a segment
  // the workgroup's element offsets inside one segment stay below 2^31 bytes
  const int64_t es = static_cast<int64_t>(elem_size(dtype));
  if (max_q * std::max(ldq, ldo) * es > INT32_MAX || max_k * std::max(ldk, ldv) * es > INT32_MAX)
    return MGATTN_ERR_SIZE;
  if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
        reinterpret_cast<uintptr_t>(out)) & 15u) != 0)
    return MGATTN_ERR_ALIGN;
  const size_t bo = span_bytes(Tq, ldo, H, d, dtype);
  if (overlaps(out, bo, q, span_bytes(Tq, ldq, H, d, dtype)) || overlaps(out, bo, k, span_bytes(Tk, ldk, Hkv, d, dtype)) ||
      overlaps(out, bo, v, span_bytes(Tk, ldv, Hkv, d, dtype)))
    return MGATTN_ERR_ALIAS;
  return MGATTN_OK;
}

// gfx950 check, cached per device ordinal (atomic entries: callers on several host
// threads may race to fill one; they all store the same value).
int device_ok() {
  static std::atomic<int> cache[64];  // 0 unknown, 1 yes, 2 no
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= 64) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    c = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c == 1;
}

template <typename Kern>
int launch_all(Kern kern, int threads, const std::vector<Launch>& plan, KernelArgs args, hipStream_t stream) {
  for (const Launch& l : plan) {
    args.table = l.table;
    void* params[] = {&args};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(static_cast<unsigned>(l.grid)),
                                         dim3(threads), params, 0, stream);
    if (e != hipSuccess) return MGATTN_ERR_LAUNCH;
  }
  return MGATTN_OK;
}

// Image table of a batch of patch grids (grids: n_img pairs {gh, gw}).
int make_images(const int32_t* grids, int n_img, ImageTable* tb) {
  if (!grids) return MGATTN_ERR_NULL;
  if (n_img < 1 || n_img > kMaxImages) return MGATTN_ERR_GRID;
  memset(tb, 0, sizeof *tb);
  tb->n = n_img;
  int64_t t = 0;
  for (int i = 0; i < n_img; ++i) {
    const int32_t gh = grids[2 * i], gw = grids[2 * i + 1];
    if (gh < 1 || gw < 1) return MGATTN_ERR_GRID;
    tb->start[i] = static_cast<int32_t>(t);
    tb->gh[i] = gh;
    tb->gw[i] = gw;
    t += static_cast<int64_t>(gh) * gw;
    if (t > INT32_MAX) return MGATTN_ERR_SIZE;
  }
  tb->start[n_img] = static_cast<int32_t>(t);
  return MGATTN_OK;
}

// One-token decoding splits a (sequence, key/value head) over several workgroups when
// the launch has fewer of them than the chip has CUs: as many splits as keep the
// workgroups within one per CU (more would only add rounds), each split with at least
// one 32-key block per wave, at most 16.
constexpr int kDecodeTargetWgs = 256;
constexpr int kMaxDecodeSplit = kMaxSplit;

int decode_split_wanted(const SegTable& t, int Hkv, int window) {
  const int wgs = t.n * Hkv;
  int max_blk = 0;
  for (int j = 0; j < t.n; ++j) {
    const int vis = window > 0 ? std::min(t.klen[j], window) : t.klen[j];
    max_blk = std::max(max_blk, (vis + 31) / 32);
  }
  int ns = kDecodeTargetWgs / wgs;
  ns = std::min(ns, std::max(1, max_blk / DecodeTile<64>::kWaves));
  return std::max(1, std::min(ns, kMaxDecodeSplit));
}

// Workspace bytes of the partial results of one launch split nsplit ways: per
// (sequence, key/value head, split) 32 query columns of d floats plus (M, den).
size_t decode_part_bytes(const SegTable& t, int Hkv, int nsplit, int d) {
  return static_cast<size_t>(t.n) * Hkv * nsplit * 32 * (static_cast<size_t>(d) + 2) * sizeof(float);
}

// Is this call one-token decoding (served by the decode kernel)?
bool is_decode(const int32_t* cu, int n_seg, int H, int Hkv, bool pack) {
  bool decode = pack && H / Hkv <= 32;
  for (int g = 0; decode && g < n_seg; ++g) decode = cu[g + 1] - cu[g] <= 1;
  return decode;
}

// Validation, plan and launches shared by every attention entry point.
int attend(const void* q, const void* k, const void* v, void* out, int64_t ldq, int64_t ldk, int64_t ldv,
           int64_t ldo, const int32_t* cu, const int32_t* cuk, int n_seg, int H, int Hkv, int d, float scale,
           int causal, int window, int dtype, void* stream, void* ws = nullptr, size_t ws_bytes = 0,
           const KernelArgs* rope = nullptr) {
  const int st = validate(q, k, v, out, ldq, ldk, ldv, ldo, cu, cuk, n_seg, H, Hkv, d, scale, causal, window, dtype);
  if (st != MGATTN_OK) return st;
  // The general bf16 kernel packs the query heads of a key/value head into one tile's
  // rows: its tiles are per key/value head, H/Hkv rows per token.
  const bool general = cuk != nullptr || Hkv != H || window != 0;
  const bool pack = general && dtype == MGATTN_BF16;
  const int H_tiles = pack ? Hkv : H;
  const DenseKind kind = general ? DenseKind::kOther : dense_kind(cu, n_seg, H, d, dtype, causal);
  const int bm = general ? block_m_of(d, dtype) : dense_block_m(cu, n_seg, H, d, dtype, causal);
  std::vector<Launch> plan;
  if (!make_plan(cu, cuk, n_seg, H_tiles, bm, plan, pack ? H / Hkv : 1)) return MGATTN_ERR_SIZE;
  if (!device_ok()) return MGATTN_ERR_DEVICE;

  KernelArgs args;
  memset(&args, 0, sizeof args);
  args.q = q;
  args.k = k;
  args.v = v;
  args.o = out;
  args.H = H_tiles;
  args.causal = causal;
  args.ldq = static_cast<int32_t>(ldq);
  args.ldk = static_cast<int32_t>(ldk);
  args.ldv = static_cast<int32_t>(ldv);
  args.ldo = static_cast<int32_t>(ldo);
  args.hq_per_kv = H / Hkv;
  args.window = window;
  // c = |scale| * log2(e) multiplies the scores inside exp2; the sign of scale goes
  // into Q (exact).  For scale == 0 the scores vanish (Q * 0) and c = 1 keeps masked
  // keys at exp2(-inf) = 0.
  args.c = scale == 0.0f ? 1.0f : static_cast<float>(fabs(static_cast<double>(scale)) * 1.4426950408889634);
  args.qsign = scale > 0.0f ? 1 : (scale < 0.0f ? -1 : 0);
  if (rope) args.rope = rope->rope;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // One-token decoding (every sequence has a single new query): the key-split decode
  // kernel, nsplit workgroups per (sequence, key/value head); nsplit > 1 only with a
  // caller's workspace large enough for the partial results, merged by a second
  // kernel.  Launches run in stream order, so each reuses the workspace.
  if (is_decode(cu, n_seg, H, Hkv, pack)) {
    for (const Launch& l : plan) {
      args.table = l.table;
      int ns = ws ? decode_split_wanted(l.table, Hkv, window) : 1;
      while (ns > 1 && decode_part_bytes(l.table, Hkv, ns, d) > ws_bytes) --ns;
      args.nsplit = ns;
      args.part = ns > 1 ? static_cast<float*>(ws) : nullptr;
      void* params[] = {&args};
      // groups of up to 16 query heads: the 16-column tile (no zero columns)
      const bool g16 = H / Hkv <= 16;
      const void* kern =
          g16 ? (d == 64 ? reinterpret_cast<const void*>(attn_decode_bf16_g16<64>)
                : d == 96 ? reinterpret_cast<const void*>(attn_decode_bf16_g16<96>)
                          : reinterpret_cast<const void*>(attn_decode_bf16_g16<128>))
              : (d == 64 ? reinterpret_cast<const void*>(attn_decode_bf16<64>)
                 : d == 96 ? reinterpret_cast<const void*>(attn_decode_bf16<96>)
                           : reinterpret_cast<const void*>(attn_decode_bf16<128>));
      const unsigned wgs = static_cast<unsigned>(l.table.n * Hkv);
      if (hipLaunchKernel(kern, dim3(wgs * ns), dim3(DecodeTile<96>::kThreads), params, 0, s) != hipSuccess)
        return MGATTN_ERR_LAUNCH;
      if (ns > 1) {
        const void* comb = d == 64 ? reinterpret_cast<const void*>(attn_decode_combine<64>)
                           : d == 96 ? reinterpret_cast<const void*>(attn_decode_combine<96>)
                                     : reinterpret_cast<const void*>(attn_decode_combine<128>);
        if (hipLaunchKernel(comb, dim3(wgs), dim3(256), params, 0, s) != hipSuccess) return MGATTN_ERR_LAUNCH;
      }
    }
    return MGATTN_OK;
  }
  if (dtype == MGATTN_BF16) {
    switch (d) {
      case 64:
        return general ? launch_all(attn_fwd_bf16<64, true>, Bf16Tile<64>::kThreads, plan, args, s)
                       : launch_all(attn_fwd_bf16<64, false>, Bf16Tile<64>::kThreads, plan, args, s);
      case 96:
        if (general) return launch_all(attn_fwd_bf16<96, true>, Bf16Tile<96>::kThreads, plan, args, s);
        switch (kind) {
          case DenseKind::kFull8:
            return rope ? launch_all(attn_fwd_bf16_pipe<96, 8, true>, 8 * 64, plan, args, s)
                        : launch_all(attn_fwd_bf16_pipe<96, 8>, 8 * 64, plan, args, s);
          case DenseKind::kFull4:
            return rope ? launch_all(attn_fwd_bf16_pipe<96, 4, true>, 4 * 64, plan, args, s)
                        : launch_all(attn_fwd_bf16_pipe<96, 4>, 4 * 64, plan, args, s);
          case DenseKind::kSplit8:
            return rope ? launch_all(attn_fwd_bf16_pipe<96, 8, true, 2>, 8 * 64, plan, args, s)
                        : launch_all(attn_fwd_bf16_pipe<96, 8, false, 2>, 8 * 64, plan, args, s);
          case DenseKind::kQuad8:
            return rope ? launch_all(attn_fwd_bf16_pipe<96, 8, true, 4>, 8 * 64, plan, args, s)
                        : launch_all(attn_fwd_bf16_pipe<96, 8, false, 4>, 8 * 64, plan, args, s);
          default: return MGATTN_ERR_HEAD_DIM;
        }
      case 128:
        return general ? launch_all(attn_fwd_bf16<128, true>, Bf16Tile<128>::kThreads, plan, args, s)
                       : launch_all(attn_fwd_bf16<128, false>, Bf16Tile<128>::kThreads, plan, args, s);
    }
  } else {
    if (kind == DenseKind::kF32Split16) {
      switch (d) {
        case 64: return launch_all(attn_fwd_f32_split16<64, f32_split16_waves<64>()>, 64 * 8, plan, args, s);
        case 96: return launch_all(attn_fwd_f32_split16<96, f32_split16_waves<96>()>, 64 * 8, plan, args, s);
        case 128: return launch_all(attn_fwd_f32_split16<128, f32_split16_waves<128>()>, 64 * 8, plan, args, s);
      }
    }
    if (kind == DenseKind::kF32Split) {
      switch (d) {
        case 64: return launch_all(attn_fwd_f32_split<64, f32_split_waves<64>()>, f32_split_waves<64>() * 64, plan, args, s);
        case 96: return launch_all(attn_fwd_f32_split<96, f32_split_waves<96>()>, f32_split_waves<96>() * 64, plan, args, s);
        case 128:
          return launch_all(attn_fwd_f32_split<128, f32_split_waves<128>()>, f32_split_waves<128>() * 64, plan, args, s);
      }
    }
    switch (d) {
      case 64: return launch_all(attn_fwd_f32<64>, F32Tile<64>::kThreads, plan, args, s);
      case 96: return launch_all(attn_fwd_f32<96>, F32Tile<96>::kThreads, plan, args, s);
      case 128: return launch_all(attn_fwd_f32<128>, F32Tile<128>::kThreads, plan, args, s);
    }
  }
  return MGATTN_ERR_HEAD_DIM;
}

// ---- scratch of mgattn_attention_kv_noalloc: the partial results of the decode key
// splits live in a file-scope device array instead of a caller's workspace.  Each
// GPU the library runs on holds its own copy until the process ends; host code only
// ever passes the device address found by hipGetSymbolAddress on that device.
// Size: the split rule keeps (sequence, key/value head, split) triples within
// kDecodeTargetWgs per launch, each writing 32 query columns of d + 2 floats, so no
// call needs more than 256 x 32 x 130 x 4 bytes = 4.06 MiB at head_dim 128; the entry
// point still refuses a larger need by name.
constexpr size_t kScratchBytes = size_t(kDecodeTargetWgs) * 32 * (128 + 2) * sizeof(float);
constexpr int kMaxDevices = 64;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch (resolved once per device), or NULL.
void* scratch_device_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" {

int mgattn_dense_strided(const void* q, const void* k, const void* v, void* out, int64_t ldq, int64_t ldk,
                         int64_t ldv, int64_t ldo, const int32_t* cu_seqlens, int n_seg, int H, int d, float scale,
                         int causal, int dtype, void* stream) {
  return attend(q, k, v, out, ldq, ldk, ldv, ldo, cu_seqlens, nullptr, n_seg, H, H, d, scale, causal, 0, dtype,
                stream);
}

int mgattn_attention_kv(const void* q, const void* k, const void* v, void* out, int64_t ldq, int64_t ldk,
                        int64_t ldv, int64_t ldo, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int n_seq, int Hq, int Hkv, int d, float scale, int window, int dtype, void* stream) {
  if (!cu_seqlens_k) return MGATTN_ERR_NULL;
  return attend(q, k, v, out, ldq, ldk, ldv, ldo, cu_seqlens_q, cu_seqlens_k, n_seq, Hq, Hkv, d, scale, 1, window,
                dtype, stream);
}

int mgattn_attention_kv_noalloc(const void* q, const void* k, const void* v, void* out, int64_t ldq, int64_t ldk,
                                int64_t ldv, int64_t ldo, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int n_seq, int Hq, int Hkv, int d, float scale, int window, int dtype, void* stream) {
  const long need = mgattn_attention_kv_workspace(cu_seqlens_q, cu_seqlens_k, n_seq, Hq, Hkv, d, window, dtype);
  if (need < 0) return static_cast<int>(need);
  if (static_cast<size_t>(need) > kScratchBytes) return MGATTN_ERR_SCRATCH;
  if (need == 0)
    return mgattn_attention_kv(q, k, v, out, ldq, ldk, ldv, ldo, cu_seqlens_q, cu_seqlens_k, n_seq, Hq, Hkv, d, scale,
                               window, dtype, stream);
  const int st = validate(q, k, v, out, ldq, ldk, ldv, ldo, cu_seqlens_q, cu_seqlens_k, n_seq, Hq, Hkv, d, scale, 1,
                          window, dtype);
  if (st != MGATTN_OK) return st;
  if (!device_ok()) return MGATTN_ERR_DEVICE;
  void* ws = scratch_device_ptr();
  if (!ws) return MGATTN_ERR_DEVICE;
  return attend(q, k, v, out, ldq, ldk, ldv, ldo, cu_seqlens_q, cu_seqlens_k, n_seq, Hq, Hkv, d, scale, 1, window,
                dtype, stream, ws, static_cast<size_t>(need));
}

long mgattn_attention_kv_noalloc_scratch_bytes(void) { return static_cast<long>(kScratchBytes); }

long mgattn_attention_kv_workspace(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seq, int Hq,
                                   int Hkv, int d, int window, int dtype) {
  if (!cu_seqlens_q || !cu_seqlens_k) return MGATTN_ERR_NULL;
  if (!dtype_ok(dtype)) return MGATTN_ERR_DTYPE;
  if (n_seq < 1) return MGATTN_ERR_SEGMENTS;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return MGATTN_ERR_HEADS;
  if (!head_dim_ok(d)) return MGATTN_ERR_HEAD_DIM;
  if (window < 0) return MGATTN_ERR_WINDOW;
  int64_t Tq = 0, Tk = 0, mq = 0, mk = 0;
  int st = check_seqlens(cu_seqlens_q, n_seq, &Tq, &mq);
  if (st != MGATTN_OK) return st;
  st = check_seqlens(cu_seqlens_k, n_seq, &Tk, &mk);
  if (st != MGATTN_OK) return st;
  for (int g = 0; g < n_seq; ++g)
    if (cu_seqlens_k[g + 1] - cu_seqlens_k[g] < cu_seqlens_q[g + 1] - cu_seqlens_q[g]) return MGATTN_ERR_SEQLENS;
  if (!is_decode(cu_seqlens_q, n_seq, Hq, Hkv, dtype == MGATTN_BF16)) return 0;
  std::vector<Launch> plan;
  if (!make_plan(cu_seqlens_q, cu_seqlens_k, n_seq, Hkv, block_m_of(d, dtype), plan, Hq / Hkv)) return MGATTN_ERR_SIZE;
  size_t need = 0;
  for (const Launch& l : plan) {
    const int ns = decode_split_wanted(l.table, Hkv, window);
    if (ns > 1) need = std::max(need, decode_part_bytes(l.table, Hkv, ns, d));
  }
  return static_cast<long>(need);
}

int mgattn_attention_kv_ws(const void* q, const void* k, const void* v, void* out, int64_t ldq, int64_t ldk,
                           int64_t ldv, int64_t ldo, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int n_seq, int Hq, int Hkv, int d, float scale, int window, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!cu_seqlens_k || (workspace_bytes > 0 && !workspace)) return MGATTN_ERR_NULL;
  if (workspace_bytes == 0)
    return attend(q, k, v, out, ldq, ldk, ldv, ldo, cu_seqlens_q, cu_seqlens_k, n_seq, Hq, Hkv, d, scale, 1, window,
                  dtype, stream);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MGATTN_ERR_ALIGN;
  const int st = validate(q, k, v, out, ldq, ldk, ldv, ldo, cu_seqlens_q, cu_seqlens_k, n_seq, Hq, Hkv, d, scale, 1,
                          window, dtype);
  if (st != MGATTN_OK) return st;
  // the workspace may not share bytes with any tensor
  const int64_t Tq = cu_seqlens_q[n_seq], Tk = cu_seqlens_k[n_seq];
  if (overlaps(workspace, workspace_bytes, q, span_bytes(Tq, ldq, Hq, d, dtype)) ||
      overlaps(workspace, workspace_bytes, out, span_bytes(Tq, ldo, Hq, d, dtype)) ||
      overlaps(workspace, workspace_bytes, k, span_bytes(Tk, ldk, Hkv, d, dtype)) ||
      overlaps(workspace, workspace_bytes, v, span_bytes(Tk, ldv, Hkv, d, dtype)))
    return MGATTN_ERR_ALIAS;
  return attend(q, k, v, out, ldq, ldk, ldv, ldo, cu_seqlens_q, cu_seqlens_k, n_seq, Hq, Hkv, d, scale, 1, window,
                dtype, stream, workspace, workspace_bytes);
}

int mgattn_dense(const void* q, const void* k, const void* v, void* out, const int32_t* cu_seqlens,
                 int n_seg, int H, int d, float scale, int causal, int dtype, void* stream) {
  const int64_t row = static_cast<int64_t>(H) * d;
  return mgattn_dense_strided(q, k, v, out, row, row, row, row, cu_seqlens, n_seg, H, d, scale, causal, dtype,
                              stream);
}

const char* mgattn_strerror(int status) {
  switch (status) {
    case MGATTN_OK: return "ok";
    case MGATTN_ERR_NULL: return "a required pointer (q, k, v, out or cu_seqlens) is NULL";
    case MGATTN_ERR_DTYPE: return "dtype is not MGATTN_F32 or MGATTN_BF16";
    case MGATTN_ERR_HEAD_DIM: return "head_dim not supported (supported: 64, 96, 128)";
    case MGATTN_ERR_HEADS: return "heads must be >= 1 (and Hq a multiple of Hkv)";
    case MGATTN_ERR_SEQLENS:
      return "cu_seqlens must start at 0, be non-decreasing and end at T > 0";
    case MGATTN_ERR_SEGMENTS: return "n_seg must be >= 1";
    case MGATTN_ERR_ALIAS: return "out overlaps q, k or v";
    case MGATTN_ERR_ALIGN: return "q, k, v and out must be 16-byte aligned";
    case MGATTN_ERR_SCALE: return "scale must be finite and causal must be 0 or 1";
    case MGATTN_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    case MGATTN_ERR_DEVICE: return "the current device is not a gfx950 (MI355X) GPU";
    case MGATTN_ERR_SIZE: return "a segment spans more than 2^31 bytes, or the grid is too large";
    case MGATTN_ERR_WINDOW: return "window must be >= 0";
    case MGATTN_ERR_SCRATCH: return "the call needs more scratch than mgattn_attention_kv_noalloc holds "
                                    "(mgattn_attention_kv_noalloc_scratch_bytes); use mgattn_attention_kv_ws";
    case MGATTN_ERR_GRID:
      return "a patch grid is empty, more than 64 images, a window below 1, or inverse not 0 or 1";
    case MGATTN_ERR_STRIDE:
      return "a leading dimension is below H*d, above 2^31-1, or not a multiple of 16 bytes";
  }
  return "unknown mgattn status";
}

int mgattn_dense_supported(int H, int d, int dtype) {
  return (H >= 1 && head_dim_ok(d) && dtype_ok(dtype)) ? 1 : 0;
}

long mgattn_dense_lds_bytes(int d, int dtype) {
  if (!dtype_ok(dtype)) return MGATTN_ERR_DTYPE;
  return lds_bytes_of(d, dtype);
}

int mgattn_dense_block_m(int d, int dtype) {
  if (!dtype_ok(dtype)) return MGATTN_ERR_DTYPE;
  if (!head_dim_ok(d)) return MGATTN_ERR_HEAD_DIM;
  return block_m_of(d, dtype);
}

int mgattn_dense_plan_block_m(const int32_t* cu_seqlens, int n_seg, int H, int d, int dtype, int causal) {
  const int nl = mgattn_dense_plan(cu_seqlens, n_seg, H, d, dtype, causal, nullptr, 0);
  if (nl < 0) return nl;
  return dense_block_m(cu_seqlens, n_seg, H, d, dtype, causal);
}

int mgattn_dense_plan(const int32_t* cu_seqlens, int n_seg, int H, int d, int dtype, int causal,
                      int64_t* grids, int max_launches) {
  if (!dtype_ok(dtype)) return MGATTN_ERR_DTYPE;
  if (!cu_seqlens) return MGATTN_ERR_NULL;
  if (n_seg < 1) return MGATTN_ERR_SEGMENTS;
  if (H < 1) return MGATTN_ERR_HEADS;
  if (!head_dim_ok(d)) return MGATTN_ERR_HEAD_DIM;
  if (causal != 0 && causal != 1) return MGATTN_ERR_SCALE;
  if (cu_seqlens[0] != 0) return MGATTN_ERR_SEQLENS;
  for (int g = 0; g < n_seg; ++g)
    if (cu_seqlens[g + 1] < cu_seqlens[g]) return MGATTN_ERR_SEQLENS;
  if (cu_seqlens[n_seg] <= 0) return MGATTN_ERR_SEQLENS;
  std::vector<Launch> plan;
  if (!make_plan(cu_seqlens, nullptr, n_seg, H, dense_block_m(cu_seqlens, n_seg, H, d, dtype, causal), plan))
    return MGATTN_ERR_SIZE;
  for (int i = 0; i < static_cast<int>(plan.size()) && i < max_launches; ++i)
    if (grids) grids[i] = plan[i].grid;
  return static_cast<int>(plan.size());
}

int mgattn_dense_tile(const int32_t* cu_seqlens, int n_seg, int H, int d, int dtype, int causal,
                      int launch, int64_t block, int32_t* seg_head_q0) {
  if (!seg_head_q0) return MGATTN_ERR_NULL;
  const int nl = mgattn_dense_plan(cu_seqlens, n_seg, H, d, dtype, causal, nullptr, 0);
  if (nl < 0) return nl;
  std::vector<Launch> plan;
  const int bm = dense_block_m(cu_seqlens, n_seg, H, d, dtype, causal);
  make_plan(cu_seqlens, nullptr, n_seg, H, bm, plan);
  if (launch < 0 || launch >= nl || block < 0 || block >= plan[launch].grid) return MGATTN_ERR_SIZE;
  const Tile t = decode_tile(plan[launch].table, H, bm, causal, static_cast<int>(block));
  if (!t.valid) return 0;
  seg_head_q0[0] = plan[launch].orig[t.slot];
  seg_head_q0[1] = t.head;
  seg_head_q0[2] = t.q0;
  return 1;
}

int mgattn_window_segments(const int32_t* grids, int n_img, int win, int32_t* cu_seqlens, int max_seg) {
  ImageTable tb;
  const int st = make_images(grids, n_img, &tb);
  if (st != MGATTN_OK) return st;
  if (win < 1) return MGATTN_ERR_GRID;
  int64_t n_seg = 0;
  for (int i = 0; i < n_img; ++i)
    n_seg += static_cast<int64_t>((tb.gh[i] + win - 1) / win) * ((tb.gw[i] + win - 1) / win);
  if (n_seg > INT32_MAX - 1) return MGATTN_ERR_SIZE;
  if (!cu_seqlens) return static_cast<int>(n_seg);
  if (max_seg < n_seg) return MGATTN_ERR_SIZE;
  int g = 0;
  cu_seqlens[0] = 0;
  for (int i = 0; i < n_img; ++i) {
    const int gh = tb.gh[i], gw = tb.gw[i];
    for (int y0 = 0; y0 < gh; y0 += win)
      for (int x0 = 0; x0 < gw; x0 += win) {
        cu_seqlens[g + 1] = cu_seqlens[g] + std::min(win, gh - y0) * std::min(win, gw - x0);
        ++g;
      }
  }
  return static_cast<int>(n_seg);
}

int mgattn_window_permute(const void* src, void* dst, int64_t row_bytes, const int32_t* grids, int n_img,
                          int win, int inverse, void* stream) {
  if (!src || !dst) return MGATTN_ERR_NULL;
  ImageTable tb;
  const int st = make_images(grids, n_img, &tb);
  if (st != MGATTN_OK) return st;
  if (win < 1 || (inverse != 0 && inverse != 1)) return MGATTN_ERR_GRID;
  if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes / 16 > INT32_MAX) return MGATTN_ERR_STRIDE;
  if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) != 0) return MGATTN_ERR_ALIGN;
  const int64_t T = tb.start[n_img];
  const size_t bytes = static_cast<size_t>(T) * static_cast<size_t>(row_bytes);
  if (overlaps(src, bytes, dst, bytes)) return MGATTN_ERR_ALIAS;
  // one wave per row, four rows per workgroup
  const unsigned grid = static_cast<unsigned>((T + 3) / 4);
  if (!device_ok()) return MGATTN_ERR_DEVICE;
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = static_cast<uint4*>(dst);
  int32_t ppr = static_cast<int32_t>(row_bytes / 16), w = win, inv = inverse, rows = static_cast<int32_t>(T);
  void* params[] = {&s, &d, &ppr, &w, &inv, &rows, &tb};
  return hipLaunchKernel(reinterpret_cast<const void*>(window_permute_kernel), dim3(grid), dim3(256), params, 0,
                         static_cast<hipStream_t>(stream)) == hipSuccess
             ? MGATTN_OK
             : MGATTN_ERR_LAUNCH;
}

int mgattn_rope2d(void* x, int64_t ldx, const int32_t* grids, int n_img, int win, int H, int d, float theta,
                  int dtype, void* stream) {
  if (!x) return MGATTN_ERR_NULL;
  if (!dtype_ok(dtype)) return MGATTN_ERR_DTYPE;
  ImageTable tb;
  const int st = make_images(grids, n_img, &tb);
  if (st != MGATTN_OK) return st;
  if (win < 0) return MGATTN_ERR_GRID;
  if (H < 1) return MGATTN_ERR_HEADS;
  if (d < 16 || d > 128 || d % 16 != 0) return MGATTN_ERR_HEAD_DIM;
  if (!(theta > 1.0f) || !isfinite(theta)) return MGATTN_ERR_SCALE;
  const int64_t row = static_cast<int64_t>(H) * d;
  if (ldx < row || ldx > INT32_MAX || ldx % (16 / static_cast<int64_t>(elem_size(dtype))) != 0)
    return MGATTN_ERR_STRIDE;
  if ((reinterpret_cast<uintptr_t>(x) & 15u) != 0) return MGATTN_ERR_ALIGN;
  RopeArgs a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.ld = ldx;
  a.H = H;
  a.d = d;
  a.win = win;
  a.pieces = static_cast<int32_t>(static_cast<int64_t>(d) * static_cast<int64_t>(elem_size(dtype)) / 16);
  for (int i = 0; i < d / 4; ++i)
    a.inv_freq[i] = static_cast<float>(pow(static_cast<double>(theta), -4.0 * i / d));
  a.tb = tb;
  // one wave per token, four tokens per workgroup (tokens < 2^31: make_images)
  int32_t n_tokens = tb.start[n_img];
  const unsigned grid = static_cast<unsigned>((static_cast<int64_t>(n_tokens) + 3) / 4);
  if (!device_ok()) return MGATTN_ERR_DEVICE;
  void* params[] = {&a, &n_tokens};
  const void* kern = dtype == MGATTN_BF16 ? reinterpret_cast<const void*>(rope2d_kernel<__bf16>)
                                          : reinterpret_cast<const void*>(rope2d_kernel<float>);
  return hipLaunchKernel(kern, dim3(grid), dim3(256), params, 0, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MGATTN_OK
             : MGATTN_ERR_LAUNCH;
}

int mgattn_dense_rope2d(const void* q, void* k, const void* v, void* out, int64_t ldq, int64_t ldk, int64_t ldv,
                        int64_t ldo, const int32_t* cu_seqlens, int n_seg, int H, int d, float scale, int causal,
                        int dtype, const int32_t* grids, int n_img, int win, float theta, void* stream) {
  if (!dtype_ok(dtype)) return MGATTN_ERR_DTYPE;
  if (!head_dim_ok(d)) return MGATTN_ERR_HEAD_DIM;
  if (dtype != MGATTN_BF16) return MGATTN_ERR_DTYPE;  // the fused path is the bf16 tower's
  if (d != 96) return MGATTN_ERR_HEAD_DIM;
  const int st = validate(q, k, v, out, ldq, ldk, ldv, ldo, cu_seqlens, nullptr, n_seg, H, H, d, scale, causal, 0,
                          dtype);
  if (st != MGATTN_OK) return st;
  KernelArgs r;
  memset(&r, 0, sizeof r);
  const int sti = make_images(grids, n_img, &r.rope.tb);
  if (sti != MGATTN_OK) return sti;
  if (win < 0) return MGATTN_ERR_GRID;
  if (r.rope.tb.start[n_img] != cu_seqlens[n_seg]) return MGATTN_ERR_GRID;  // the images hold the call's tokens
  if (!(theta > 1.0f) || !isfinite(theta)) return MGATTN_ERR_SCALE;
  r.rope.win = win;
  for (int i = 0; i < d / 4; ++i)
    r.rope.inv_freq[i] = static_cast<float>(pow(static_cast<double>(theta), -4.0 * i / d));
  // k rotated in place by the RoPE pass, then the attention rotates q as it reads it
  const int stk = mgattn_rope2d(k, ldk, grids, n_img, win, H, d, theta, dtype, stream);
  if (stk != MGATTN_OK) return stk;
  return attend(q, k, v, out, ldq, ldk, ldv, ldo, cu_seqlens, nullptr, n_seg, H, H, d, scale, causal, 0, dtype,
                stream, nullptr, 0, &r);
}

int mgattn_version(void) { return kVersion; }

}  // extern "C"
