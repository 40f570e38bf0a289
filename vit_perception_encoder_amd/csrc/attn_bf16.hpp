// Single-pass online-softmax attention, bf16 inputs, f32 accumulation, gfx950.
//
// What it computes is the segmented softmax attention of the Muse Glimmer vision
// tower (vllm.cpp issue #1545, sections "Why this one is bad" and "The fix"): each
// segment of cu_seqlens is attended on its own, non-causal unless asked.  The flash
// rung the pages route the tower to (PR #1579, "Numerics, both halves") reaches the
// same function with a running online softmax; this kernel does too, designed for
// CDNA4 rather than after that CUDA kernel.
//
// One workgroup = 8 waves = one (segment, head, 256-query tile).
//   * Each wave owns 32 queries.  Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K is the A operand (keys are MFMA rows), Q^T the B
//     operand (queries are MFMA columns).  In the 32x32 accumulator a lane then holds
//     ONE query and 16 of the 32 keys (rows 8*(r/4) + 4*(lane/32) + r%4), so the row
//     max and row sum are in-lane chains plus one exchange between lanes l and l^32
//     (v_permlane32_swap).  head_dim is the contraction: D/16 MFMA steps (96 = 6x16).
//   * O^T = V^T P^T, again 32x32x16: P^T is the B operand and is exactly the 8
//     probabilities a lane already holds for one 16-key group, converted to bf16 in
//     place (no cross-lane shuffle).  The V^T A operand is read from a row-major V
//     tile with two ds_read_b64_tr_b16 (the LDS transpose read: within 16 lanes,
//     lane i gets element i%4 of the 8 bytes addressed by lanes 4j + i/4, j = 0..3),
//     addressed so each lane receives 4 keys of its own channel.  O^T is D/32
//     accumulators of 32x32 (96 = 3 x 32).
//   * K/V tiles of 128 keys go HBM -> LDS by LDS DMA (global_load_lds_dwordx4: each
//     lane's 16 bytes land at M0 + 16*lane, no registers involved) into three LDS
//     stages (two for head_dim 128), issued two phases before they are published.
//     The K operands of the next QK product are read from LDS during the softmax
//     phase (at head_dim 128 the first half of them; the rest at the start of the
//     MFMA phase), so the MFMA phase issues its QK MFMAs back to back.
//     K rows are padded by one 16-byte slot (D/8 + 1 slots: 208 B at head_dim 96;
//     every 16-byte MFMA operand read is free of bank conflicts); the padding slot of a
//     row receives a second copy of its last 16 bytes, so every DMA lane is active.
//   * Softmax (per 64-key step) uses exp2 with scale*log2(e) folded into one FMA per
//     score.  The running maximum is refreshed only when a step's maximum exceeds it
//     by more than 2^8 in probability terms (decided per wave), so the O rescale is
//     skipped on almost every step; exact, because numerator and denominator share
//     the reference.  The row sum adds the bf16-rounded probabilities that feed the
//     PV product (v_dot2 with ones), so the weights stay normalised.
//   * Ping-pong: waves 0-3 and 4-7 share SIMDs pairwise and run the same sequence of
//     MFMA phases (PV of the previous step + QK of the next, 24 MFMAs) and VALU phases
//     (softmax) one phase apart, with a workgroup barrier closing every phase; so
//     each SIMD always has one wave feeding the matrix core and one on the VALU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "plan.hpp"
#include "schedule.hpp"
#include "window_rope.hpp"

namespace mgattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct KernelArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int32_t H;
  int32_t causal;
  float c;        // |scale| * log2(e), or 1 when scale == 0 (always > 0)
  int32_t qsign;  // sign of scale: Q is multiplied by +1, -1 or 0 in registers (exact)
  int32_t ldq, ldk, ldv, ldo;  // elements between consecutive tokens of q, k, v, out
  int32_t hq_per_kv;  // query heads per key/value head (1 without grouping)
  int32_t window;     // causal sliding window in keys, the query's own included (0: none)
  int32_t nsplit;     // one-token decoding: workgroups per (sequence, key/value head)
  float* part;        // nsplit > 1: partial results of the key splits (caller's workspace)
  SegTable table;
  // 2D RoPE of Q on load (mgattn_dense_rope2d): batch tokens in raster or window order
  // over the images of tb, pair frequencies inv_freq[i] = theta^(-4i/d)
  struct {
    int32_t win;
    float inv_freq[32];
    ImageTable tb;
  } rope;
};
static_assert(sizeof(KernelArgs) <= 4096, "kernel arguments must stay within 4 KB");

template <int D>
struct Bf16Tile : sched::Geometry<D> {
  using G = sched::Geometry<D>;
  static constexpr int kWaves = 8;
  static constexpr int kQBlocks = 1;                     // 32-query blocks per wave
  static constexpr int kBlockM = kWaves * kQBlocks * 32; // queries per workgroup
  static constexpr int kThreads = kWaves * 64;
  static_assert(D % 32 == 0 && D >= 32 && D <= 128, "head_dim must be a multiple of 32 up to 128");
  static_assert(G::kBlockN % G::kStepKeys == 0 && G::kStepKeys % 32 == 0, "LDS tile must hold whole softmax steps");
  static_assert((G::kBlockN * D / 8) % 64 == 0, "V tile must be whole DMA instructions");
  static_assert(G::kKElems % 8 == 0 && G::kStageElems % 8 == 0, "LDS regions must stay 16-byte aligned");
  static_assert(G::kBlockN * G::kKSlots % 64 == 0, "K tile must be whole DMA instructions");
};

// Exchange with lane l^32 and combine (max or sum) -- one v_permlane32_swap.
__device__ inline float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Exchange with lane l^16 and combine (max or sum) -- one v_permlane16_swap: rows of 16
// lanes 0 <-> 1 and 2 <-> 3.
__device__ inline float row16_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float row16_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key (relative to the 32-key block) held in accumulator register r by lane half hf.
__device__ constexpr int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

typedef __bf16 bf16x4_raw __attribute__((__vector_size__(4 * sizeof(__bf16))));
#define MGATTN_LDS __attribute__((address_space(3)))

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((MGATTN_LDS const void*)p));
}

// LDS DMA of 16 bytes per active lane: lane l's bytes at g land at LDS address
// m0 + 16*l.  Written as asm (no output registers; the address is read at issue) so
// that the compiler does not order later LDS reads behind it: the one wait for the
// DMA is the explicit vmcnt(0) before the barrier that publishes the tile.
// M0 is not named as clobbered: LLVM reserves M0 and does not honour a clobber of a
// reserved register.  These kernels make no other use of M0 (no LDS-DMA builtin,
// interpolation, message or indexed lane access), which a host test checks on the
// generated gfx950 assembly: every M0 write is the one inside these asm statements.
__device__ inline void dma16(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(g) : "memory");
}
// The same with a wave-uniform base and a per-lane 32-bit byte offset (the scalar-base
// form): no per-lane 64-bit address arithmetic at issue.
// The base is passed through readfirstlane: it is wave-uniform by construction, and the
// "s" constraint is only honoured for values the compiler also proves uniform.
__device__ inline void dma16s(const void* base, uint32_t off, uint32_t m0) {
  // (readfirstlane returns a signed int: each half goes back to uint32_t before it is
  // widened, or bit 31 of the low half would be sign-extended into the high half)
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint64_t bs = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(off), "s"(bs) : "memory");
}
__device__ inline void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most n (wave-uniform) of this wave's vector-memory operations are
// outstanding: they complete in issue order, so the older ones are done.  Counts above
// 63 (the counter's range) wait for all.
#define MGATTN_VMCNT_CASE(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
__device__ inline void dma_wait_leave(int n) {
  switch (n) {
    MGATTN_VMCNT_CASE(1) MGATTN_VMCNT_CASE(2) MGATTN_VMCNT_CASE(3) MGATTN_VMCNT_CASE(4) MGATTN_VMCNT_CASE(5) MGATTN_VMCNT_CASE(6) MGATTN_VMCNT_CASE(7) MGATTN_VMCNT_CASE(8)
    MGATTN_VMCNT_CASE(9) MGATTN_VMCNT_CASE(10) MGATTN_VMCNT_CASE(11) MGATTN_VMCNT_CASE(12) MGATTN_VMCNT_CASE(13) MGATTN_VMCNT_CASE(14) MGATTN_VMCNT_CASE(15) MGATTN_VMCNT_CASE(16)
    MGATTN_VMCNT_CASE(17) MGATTN_VMCNT_CASE(18) MGATTN_VMCNT_CASE(19) MGATTN_VMCNT_CASE(20) MGATTN_VMCNT_CASE(21) MGATTN_VMCNT_CASE(22) MGATTN_VMCNT_CASE(23) MGATTN_VMCNT_CASE(24)
    MGATTN_VMCNT_CASE(25) MGATTN_VMCNT_CASE(26) MGATTN_VMCNT_CASE(27) MGATTN_VMCNT_CASE(28) MGATTN_VMCNT_CASE(29) MGATTN_VMCNT_CASE(30) MGATTN_VMCNT_CASE(31) MGATTN_VMCNT_CASE(32)
    MGATTN_VMCNT_CASE(33) MGATTN_VMCNT_CASE(34) MGATTN_VMCNT_CASE(35) MGATTN_VMCNT_CASE(36) MGATTN_VMCNT_CASE(37) MGATTN_VMCNT_CASE(38) MGATTN_VMCNT_CASE(39) MGATTN_VMCNT_CASE(40)
    MGATTN_VMCNT_CASE(41) MGATTN_VMCNT_CASE(42) MGATTN_VMCNT_CASE(43) MGATTN_VMCNT_CASE(44) MGATTN_VMCNT_CASE(45) MGATTN_VMCNT_CASE(46) MGATTN_VMCNT_CASE(47) MGATTN_VMCNT_CASE(48)
    MGATTN_VMCNT_CASE(49) MGATTN_VMCNT_CASE(50) MGATTN_VMCNT_CASE(51) MGATTN_VMCNT_CASE(52) MGATTN_VMCNT_CASE(53) MGATTN_VMCNT_CASE(54) MGATTN_VMCNT_CASE(55) MGATTN_VMCNT_CASE(56)
    MGATTN_VMCNT_CASE(57) MGATTN_VMCNT_CASE(58) MGATTN_VMCNT_CASE(59) MGATTN_VMCNT_CASE(60) MGATTN_VMCNT_CASE(61) MGATTN_VMCNT_CASE(62) MGATTN_VMCNT_CASE(63)
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}
#undef MGATTN_VMCNT_CASE

// LDS transpose read: 4 bf16 (see the layout note at the top of this file).
__device__ inline bf16x4 ds_read_tr(const __bf16* p) {
  const bf16x4_raw r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MGATTN_LDS bf16x4_raw*)p);
  return __builtin_bit_cast(bf16x4, r);
}

// kGeneral: keys from their own segment rows (a KV cache), grouped key/value heads and
// a sliding window are read from the arguments.  Without it (the dense entry points)
// keys are the queries, heads are not grouped and there is no window, as compile-time
// facts, so the dense kernel carries none of that arithmetic.
template <int D, bool kGeneral>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(KernelArgs a) {
  using TL = Bf16Tile<D>;
  constexpr int BM = TL::kBlockM, BN = TL::kBlockN;
  constexpr int SK = TL::kStepKeys;  // keys per softmax step
  constexpr int NB = SK / 32;        // 32-key blocks per softmax step
  constexpr int NSTEP = BN / SK;     // softmax steps per LDS tile
  constexpr int KS = D / 16;         // MFMA k-steps over head_dim
  constexpr int CT = D / 32;         // 32-channel output tiles
  constexpr int KP = TL::kKPitch, VP = TL::kVPitch, KSL = TL::kKSlots;
  constexpr int KDMA = TL::kKDma, VDMA = TL::kVDma;
  constexpr int KDMA_W = (KDMA + TL::kWaves - 1) / TL::kWaves;  // per wave (upper bound)
  constexpr int VDMA_W = (VDMA + TL::kWaves - 1) / TL::kWaves;
  constexpr float kRescaleLog2 = 8.0f;  // refresh the running max past 2^8 growth
  static_assert(TL::kQBlocks == 1, "one 32-query block per wave");
  // K operands of the next QK product are read during the softmax phase.  At
  // head_dim 128 all of them (64 registers) would spill, so only the first half of
  // the contraction's fragments is read there and the rest at the start of the MFMA
  // phase that uses them; the QK product consumes the fragments in that order.
  constexpr int kPreK = D < 128 ? KS : KS / 2;

  __shared__ __attribute__((aligned(16))) __bf16 lds[TL::kStages * TL::kStageElems];

  const Tile tile = decode_tile(a.table, a.H, BM, a.causal, blockIdx.x);
  if (!tile.valid) return;
  // Query rows.  The general instantiation packs the G query heads that share a
  // key/value head into the rows of one tile (row r = token r / G, query head
  // kvhead * G + r % G), so K and V are read once per key/value head; the dense one
  // has G = 1 and the tile's own head.
  const int G = kGeneral ? a.hq_per_kv : 1;
  const int L = a.table.len[tile.slot];                   // query tokens of the segment
  const int R = L * G;                                    // query rows
  const int Lk = kGeneral ? a.table.klen[tile.slot] : L;  // keys of the segment
  const int off = Lk - L;                                 // position of query token 0 among the keys
  const int window = kGeneral ? a.window : 0;
  const int q0 = tile.q0;                                 // first row of the tile
  // Token t, head h of a tensor with leading dimension ld starts at t*ld + h*D.
  const size_t t0 = static_cast<size_t>(a.table.start[tile.slot]);
  const size_t tk0 = kGeneral ? static_cast<size_t>(a.table.kstart[tile.slot]) : t0;
  const size_t kvoff = static_cast<size_t>(tile.head) * D;  // key/value head (= the query head when G = 1)
  auto row_offset = [&](int r, int ld) {  // offset of query row r in q or out
    const int qh = kGeneral ? tile.head * G + r % G : tile.head;
    return static_cast<size_t>(r / G) * ld + static_cast<size_t>(qh) * D;
  };
  const __bf16* __restrict__ qg = static_cast<const __bf16*>(a.q) + t0 * a.ldq;
  const __bf16* __restrict__ kg = static_cast<const __bf16*>(a.k) + tk0 * a.ldk + kvoff;
  const __bf16* __restrict__ vg = static_cast<const __bf16*>(a.v) + tk0 * a.ldv + kvoff;
  __bf16* __restrict__ og = static_cast<__bf16*>(a.o) + t0 * a.ldo;
  const int ldk = a.ldk, ldv = a.ldv;

  const int tid = threadIdx.x;
  // wave index, marked wave-uniform so branches on it are scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const float c = a.c;
  const int qr = q0 + wave * 32 + n;  // this lane's query row (relative to the segment)
  const int qmin = q0 + wave * 32;    // the wave's first row
  const int qpos = off + qr / G;      // the lane's query position among the keys

  bf16x8 qf[KS];  // Q fragments, read from LDS once the Q tile has arrived
  // Keys this q-tile needs: up to its last query token (causal), from its first
  // token's window start (whole tiles below it are skipped).  Tile 0 starts at kb0.
  const int tok_last = (min(R, q0 + BM) - 1) / G;
  const int kend = a.causal ? min(Lk, off + tok_last + 1) : Lk;
  const int kbeg = window > 0 ? max(0, off + q0 / G - window + 1) : 0;
  const int kb0 = (kbeg / BN) * BN;
  const int ntiles = (kend - kb0 + BN - 1) / BN;
  const int nsteps = (kend - kb0 + SK - 1) / SK;

  // ---- LDS DMA plan.  DMA instruction i of a tile fills 64 consecutive 16-byte
  // slots (1 KB); wave w issues instructions w, w+8, ...  K slot s is row s/KSL,
  // piece s%KSL (piece D/8 is padding: loaded from piece D/8-1).  V slot s is row s/(D/8),
  // piece s%(D/8).  Rows past the segment end are clamped to its last row: their
  // keys are masked (p = 0) and the clamped data is finite.
  int k_row[KDMA_W], k_off[KDMA_W];
#pragma unroll
  for (int u = 0; u < KDMA_W; ++u) {
    const int slot = (wave + TL::kWaves * u) * 64 + lane;
    const int row = slot / KSL, piece = slot % KSL;
    k_row[u] = row;
    k_off[u] = min(piece, D / 8 - 1) * 8;  // the padding slot gets a copy of the last piece
  }
  int v_row[VDMA_W], v_off[VDMA_W];
#pragma unroll
  for (int u = 0; u < VDMA_W; ++u) {
    const int slot = (wave + TL::kWaves * u) * 64 + lane;
    v_row[u] = slot / (D / 8);
    v_off[u] = (slot % (D / 8)) * 8;
  }
  // Byte offsets of the slots from the tile's first row, for tiles with BN valid rows
  // (every tile but a segment's last); a tile lies inside its segment, whose span is
  // below 2^31 bytes, so the offsets fit 32 bits.
  uint32_t k_boff[KDMA_W], v_boff[VDMA_W];
#pragma unroll
  for (int u = 0; u < KDMA_W; ++u)
    k_boff[u] = (static_cast<uint32_t>(k_row[u]) * static_cast<uint32_t>(ldk) + k_off[u]) * 2u;
#pragma unroll
  for (int u = 0; u < VDMA_W; ++u)
    v_boff[u] = (static_cast<uint32_t>(v_row[u]) * static_cast<uint32_t>(ldv) + v_off[u]) * 2u;
  auto issue_tile = [&](int t, int part) {  // part: 1 = K, 2 = V, 3 = both
    const int kt0 = kb0 + t * BN;
    const int last = Lk - 1 - kt0;  // last valid row of this tile (>= 0)
    const __bf16* kb = kg + static_cast<size_t>(kt0) * ldk;
    const __bf16* vb = vg + static_cast<size_t>(kt0) * ldv;
    __bf16* kl = lds + (t % TL::kStages) * TL::kStageElems;
    __bf16* vl = kl + TL::kKElems;
    if (last >= BN - 1) {  // wave-uniform: every row valid, precomputed offsets
#pragma unroll
      for (int u = 0; u < KDMA_W; ++u) {
        const int i = wave + TL::kWaves * u;
        if ((part & 1) && (KDMA % TL::kWaves == 0 || i < KDMA))
          dma16s(kb, k_boff[u], __builtin_amdgcn_readfirstlane(lds_addr(kl + i * 512)));
      }
#pragma unroll
      for (int u = 0; u < VDMA_W; ++u) {
        const int i = wave + TL::kWaves * u;
        if ((part & 2) && (VDMA % TL::kWaves == 0 || i < VDMA))
          dma16s(vb, v_boff[u], __builtin_amdgcn_readfirstlane(lds_addr(vl + i * 512)));
      }
      return;
    }
    // a segment's last tile: rows past its end are clamped to its last row
#pragma unroll
    for (int u = 0; u < KDMA_W; ++u) {
      const int i = wave + TL::kWaves * u;
      if ((part & 1) && (KDMA % TL::kWaves == 0 || i < KDMA))
        dma16(kb + static_cast<size_t>(min(k_row[u], last)) * ldk + k_off[u],
              __builtin_amdgcn_readfirstlane(lds_addr(kl + i * 512)));
    }
#pragma unroll
    for (int u = 0; u < VDMA_W; ++u) {
      const int i = wave + TL::kWaves * u;
      if ((part & 2) && (VDMA % TL::kWaves == 0 || i < VDMA))
        dma16(vb + static_cast<size_t>(min(v_row[u], last)) * ldv + v_off[u],
              __builtin_amdgcn_readfirstlane(lds_addr(vl + i * 512)));
    }
  };

  // ---- running state of this lane's query
  f32x16 o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x16{};
  float m_run = 0.0f, l_run = 0.0f;
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  f32x16 s[NB];          // scores of the current step (written by an MFMA phase)
  bf16x8 pk[NB][2];      // probabilities of the current step (written by a VALU phase)
  bf16x8 kpre[KS][NB];   // K operands of the next QK product (read during a VALU phase)

  // Where step j's keys live: LDS buffer of its tile, and its first 32-key block.
  auto step_buf = [&](int j) { return lds + ((j / NSTEP) % TL::kStages) * TL::kStageElems; };
  auto step_b = [&](int j) { return (j % NSTEP) * NB; };

  // V^T transpose-read lane addressing: lane r of each 16-lane group reads row
  // (key) r/4 (+4 for the upper lane half, +8 for the second read) at channel
  // 16*(group%2) + 4*(r%4) of the 32-channel tile.
  const int tr_row = ((lane & 15) >> 2) + 4 * hf;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // MFMA work: O^T += V^T P^T for step j, and S^T = K Q^T for step j (12 MFMAs each).
  auto mfma_pv = [&](int j) {
    const __bf16* vt = step_buf(j) + TL::kKElems;
    const int kb0 = step_b(j);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const __bf16* vrow = vt + ((kb0 + b) * 32 + h2 * 16 + tr_row) * VP + tr_col;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const bf16x4 lo = ds_read_tr(vrow + ct * 32);
          const bf16x4 hi = ds_read_tr(vrow + 8 * VP + ct * 32);
          const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk[b][h2], o[ct], 0, 0, 0);
        }
      }
  };
  auto read_k = [&](int j, int st0, int st1) {  // fragments st0 .. st1-1 of step j
    const __bf16* ks = step_buf(j);
    const int kb0 = step_b(j);
#pragma unroll
    for (int st = st0; st < st1; ++st)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        kpre[st][b] = *reinterpret_cast<const bf16x8*>(ks + ((kb0 + b) * 32 + n) * KP + 16 * st + 8 * hf);
  };
  auto mfma_qk = [&]() {
#pragma unroll
    for (int b = 0; b < NB; ++b) s[b] = f32x16{};
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int b = 0; b < NB; ++b) s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kpre[st][b], qf[st], s[b], 0, 0, 0);
  };

  // VALU phase j: online softmax of step j's scores into bf16 probabilities.  Keys
  // past the segment end and (causal) keys after the query get s = -inf, hence p = 0
  // (c is always positive).
  // General instantiation: steps j_lo .. j_hi need no mask for any row of the wave
  // (every key inside each row's window, at or before its position, before the segment
  // end), and the per-lane limits are taken relative to the lane's first key of a step,
  // so the loop keeps two step bounds and three lane values instead of the segment's
  // scalars (which would not fit the SGPRs beside the DMA state).
  const int pos_lo = off + qmin / G, pos_hi = off + (qmin + 31) / G;  // the wave's first and last positions
  int j_lo = 0, j_hi = 0, lim_end = 0, lim_causal = 0, lim_window = 0;
  if constexpr (kGeneral) {
    j_lo = window > 0 ? max(0, (pos_hi - window + 1 - kb0 + SK - 1) / SK) : 0;
    j_hi = (Lk - SK - kb0) >= 0 ? (Lk - SK - kb0) / SK : -1;
    if (a.causal) j_hi = min(j_hi, (pos_lo - SK + 1 - kb0) >= 0 ? (pos_lo - SK + 1 - kb0) / SK : -1);
    // (2^30 sentinels: key0 < 2^30 for any admitted segment, so the differences stay in
    // range; a window wider than the keys masks nothing, as does a window of Lk)
    lim_end = Lk - 4 * hf;                                                  // masked: key offset >= lim_end - key0
    lim_causal = a.causal ? qpos - 4 * hf : (1 << 30);                      // masked: offset > lim_causal - key0
    lim_window = window > 0 ? qpos - min(window, Lk) - 4 * hf : -(1 << 30);  // masked: offset <= lim_window - key0
  }
  auto valu_phase = [&](int j) {
    if (j + 1 < nsteps) read_k(j + 1, 0, kPreK);  // in flight while the softmax runs
    const int key0 = kb0 + j * SK;
    if constexpr (kGeneral) {
      if (j < j_lo || j > j_hi) {
        const int d_end = lim_end - key0, d_causal = lim_causal - key0, d_window = lim_window - key0;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kofs = b * 32 + acc_row(r, 0);  // key offset of register r from the lane's first key
            if (kofs >= d_end || kofs > d_causal || kofs <= d_window) s[b][r] = -INFINITY;
          }
      }
    } else if ((key0 + SK > Lk) || (a.causal && key0 + SK - 1 > pos_lo)) {
      const int pos = qpos;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + b * 32 + acc_row(r, hf);
          if (key >= Lk || (a.causal && key > pos)) s[b][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
    // a step with no key for some rows (outside their window) has maximum -inf; a
    // finite floor keeps the reference finite (those rows get p = 0, and the first
    // step with keys refreshes the reference with alpha = 0)
    const float m_blk = fmaxf(half_swap_max(mx), -1.0e30f);
    if (j == 0) {
      m_run = m_blk;
    } else if (__builtin_amdgcn_ballot_w64((m_blk - m_run) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m_run, m_blk);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct] *= alpha;
    }
    const float mc = m_run * c;
    float lsum = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pv[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[b][8 * h2 + e], c, -mc)));
        pk[b][h2] = pv;
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pv[e], pv[e + 1]}, ones, lsum, false);
      }
    l_run += lsum;
  };

  // Tile staging by phase.  Step j's K is read in VALU phase j-1 and its V in MFMA
  // phase j+1, so tile t (steps tN .. tN+N-1) is read in phases 2tN-1 .. 2tN+2N+1 of
  // the leading group (one later for the trailing one).  Its DMA is waited for at the
  // end of phase W(t) = 2tN-2 (published for 2tN-1) and issued at the start of phase
  // I(t) = max(2tN-4, 2N(t-S+1)+2): two phases of latency when the buffer it replaces
  // (tile t-S, last read in phase 2N(t-S+1)+1) is already free.
  constexpr int N2 = 2 * NSTEP;
  auto issue_phase = [&](int t) { return sched::phased_issue_phase(t, NSTEP, TL::kStages); };
  int t_issue = 0, t_wait = 0;
  // The workgroup's Q tile goes to the last stage by LDS DMA as well (whole rows,
  // 16 bytes per lane; rows past the segment end clamped), together with the first
  // K/V tile.  That stage receives its first tile (tile kStages-1) no earlier than
  // phase 2 (the staging rule below), after barriers that follow every wave's reads
  // of its Q fragments.  Only the leading group's Q rows and K of tile 0 are waited
  // for before the first barrier; the trailing group's Q rows and V of tile 0 (first
  // read in phases 1 and 2) are issued after them and waited for at the end of phase 0.
  constexpr int QDMA = BM * D / 8 / 64;
  constexpr int QDMA_W = QDMA / TL::kWaves;  // per wave: first half rows of waves 0-3, second half 4-7
  static_assert(QDMA % (2 * TL::kWaves) == 0 && BM * D <= TL::kStageElems, "Q tile must fit one stage");
  static_assert(VDMA % TL::kWaves == 0 && N2 - 4 >= 0, "V DMAs split evenly; only tile 0 precedes phase 0");
  __bf16* ql = lds + (TL::kStages - 1) * TL::kStageElems;
  auto issue_q = [&](int u0, int u1) {
#pragma unroll
    for (int u = 0; u < QDMA_W; ++u) {
      if (u < u0 || u >= u1) continue;
      const int i = wave + TL::kWaves * u;
      const int slot = i * 64 + lane;
      dma16(qg + row_offset(min(q0 + slot / (D / 8), R - 1), a.ldq) + (slot % (D / 8)) * 8,
            __builtin_amdgcn_readfirstlane(lds_addr(ql + i * 512)));
    }
  };
  issue_q(0, QDMA_W / 2);
  issue_tile(0, 1);
  issue_q(QDMA_W / 2, QDMA_W);
  issue_tile(0, 2);
  t_issue = 1;
  t_wait = 1;
  // With three stages a tile's V goes one phase after its K (spreading the DMA issue
  // over two phases); both are waited for at the same phase end.
  int v_pending = -1;
  dma_wait_leave(QDMA_W / 2 + VDMA / TL::kWaves);
  __syncthreads();
  // this wave's K DMAs per tile (issued in stage_begin(0) for tile 1 with three stages)
  const int my_kdma = KDMA / TL::kWaves + (wave < KDMA % TL::kWaves ? 1 : 0);

  // ---- Q fragments (B operand of S^T): lane holds query qr, channels 16s + 8hf + [0,8)
  auto read_q = [&]() {
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(ql + (wave * 32 + n) * D + 16 * s + 8 * hf);
    if (qr >= R) {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = bf16x8{};
    }
    if (a.qsign != 1) {
      const __bf16 sg = static_cast<__bf16>(static_cast<float>(a.qsign));
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = qf[s] * sg;
    }
  };
  auto stage_begin = [&](int p) {
    if (v_pending >= 0) {
      issue_tile(v_pending, 2);
      v_pending = -1;
    }
    if (t_issue < ntiles && issue_phase(t_issue) == p) {
      if (TL::kStages >= 3) {
        issue_tile(t_issue, 1);
        v_pending = t_issue;
      } else {
        issue_tile(t_issue, 3);
      }
      ++t_issue;
    }
  };
  auto stage_end = [&](int p) {
    if (p == 0) dma_wait_leave(TL::kStages >= 3 && t_issue >= 2 ? my_kdma : 0);  // Q rows 128.., V of tile 0
    if (t_wait < ntiles && sched::phased_wait_phase(t_wait, NSTEP) == p) {
      dma_wait();
      ++t_wait;
    }
  };

  // Phase schedule.  A wave's own sequence is MFMA(0), VALU(0), MFMA(1), VALU(1), ...,
  // VALU(n-1), MFMA(n): MFMA(j) is the PV product of step j-1 and the QK product of
  // step j.  Waves 0-3 run slot i in phase i; waves 4-7 (which share the SIMDs of
  // waves 0-3) run it in phase i+1.  In every phase one wave of each SIMD issues
  // MFMAs while the other runs its softmax, and a barrier closes each phase; both
  // groups pass the same 2n+2 barriers.
  const int n_st = nsteps;
  if (wave < 4) {
    read_q();
    stage_begin(0);
    read_k(0, 0, KS);
    mfma_qk();
    stage_end(0);
    __syncthreads();
    for (int j = 0; j + 1 < n_st; ++j) {
      stage_begin(2 * j + 1);
      valu_phase(j);
      stage_end(2 * j + 1);
      __syncthreads();
      stage_begin(2 * j + 2);
      if (kPreK < KS) read_k(j + 1, kPreK, KS);
      mfma_qk();
      mfma_pv(j);
      stage_end(2 * j + 2);
      __syncthreads();
    }
    stage_begin(2 * n_st - 1);
    valu_phase(n_st - 1);
    stage_end(2 * n_st - 1);
    __syncthreads();
    stage_begin(2 * n_st);
    mfma_pv(n_st - 1);
    stage_end(2 * n_st);
    __syncthreads();
    stage_begin(2 * n_st + 1);
    stage_end(2 * n_st + 1);
    __syncthreads();
  } else {
    stage_begin(0);
    stage_end(0);
    __syncthreads();
    read_q();
    stage_begin(1);
    read_k(0, 0, KS);
    mfma_qk();
    stage_end(1);
    __syncthreads();
    for (int j = 0; j + 1 < n_st; ++j) {
      stage_begin(2 * j + 2);
      valu_phase(j);
      stage_end(2 * j + 2);
      __syncthreads();
      stage_begin(2 * j + 3);
      if (kPreK < KS) read_k(j + 1, kPreK, KS);
      mfma_qk();
      mfma_pv(j);
      stage_end(2 * j + 3);
      __syncthreads();
    }
    stage_begin(2 * n_st);
    valu_phase(n_st - 1);
    stage_end(2 * n_st);
    __syncthreads();
    stage_begin(2 * n_st + 1);
    mfma_pv(n_st - 1);
    stage_end(2 * n_st + 1);
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16 (round to nearest even), rows inside the segment
  // only.  The wave's 32 x D tile is staged through its own LDS rows (every wave has
  // passed the last barrier, so the K/V stages are dead) and stored as whole rows,
  // 16 bytes per lane: in the accumulator layout a lane holds one query and 4
  // channels per register group, which would scatter 8-byte pieces over 32 rows.
  // The stores are non-temporal: no later work of this launch reads the output, and
  // lines that stay dirty in the XCDs' L2 must be written back when the kernel ends,
  // before the next launch on the stream can start (~1 us less per launch).
  const float inv = 1.0f / half_swap_sum(l_run);
  constexpr int OP = D + 8;  // O row pitch in LDS (elements), rows 16-byte aligned
  static_assert(TL::kWaves * 32 * OP <= TL::kStages * TL::kStageElems, "O staging must fit in the K/V stages");
  __bf16* ow = lds + wave * 32 * OP;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = static_cast<__bf16>(o[ct][4 * r4 + e] * inv);
      *reinterpret_cast<bf16x4*>(ow + n * OP + ct * 32 + r4 * 8 + 4 * hf) = val;
    }
  constexpr int CH = D / 8;  // 16-byte pieces per row
  constexpr int NU = 32 * CH / 64;
  static_assert(32 * CH % 64 == 0, "whole store instructions per wave");
  bf16x8 piece_val[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int cidx = u * 64 + lane;
    piece_val[u] = *reinterpret_cast<const bf16x8*>(ow + (cidx / CH) * OP + (cidx % CH) * 8);
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int cidx = u * 64 + lane;
    const int row = cidx / CH;
    if (qmin + row < R)
      __builtin_nontemporal_store(piece_val[u], reinterpret_cast<bf16x8*>(og + row_offset(qmin + row, a.ldo) + (cidx % CH) * 8));
  }
}

}  // namespace mgattn
