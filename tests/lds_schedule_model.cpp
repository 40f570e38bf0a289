// Host model of the LDS staging of the bf16 attention kernels.
//
// Every wave's program is replayed as a list of events -- DMA issue (with this wave's
// instruction count), counted wait ("at most n of my DMA instructions outstanding"),
// workgroup barrier, LDS read of an object, write of the output staging rows -- using
// the schedule functions the kernels themselves call (vit_perception_encoder_amd/csrc/
// schedule.hpp).  Epochs are counted in barriers.  A wave's DMA instructions complete
// in issue order (the vmcnt rule), so a counted wait completes exactly the older ones.
// The checks, for every wave and every case:
//   read:  an object is read only in an epoch after every wave's share of its DMA was
//          waited for (the barrier between publishes it);
//   write: a DMA into a region, or the output staging, starts only in an epoch after
//          every read of whatever occupied the region before, and after that
//          occupant's DMA completed in every wave;
//   end:   every DMA is waited for before the wave exits, and all waves pass the same
//          number of barriers.
// usage: lds_schedule_model [mutation]   (prints "ok <cases>" or the first violation)
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../vit_perception_encoder_amd/csrc/schedule.hpp"

using namespace mgattn::sched;

static const char* g_mutation = "";
static bool mutated(const char* m) { return strcmp(g_mutation, m) == 0; }

enum Kind { ISSUE, WAIT_LEAVE, BARRIER, READ, WRITE };
struct Ev {
  Kind kind;
  int obj;    // object id (ISSUE, READ, WRITE)
  int count;  // DMA instructions (ISSUE) or instructions left outstanding (WAIT_LEAVE)
};
struct Region {
  long lo, hi;  // element interval [lo, hi)
};

struct Model {
  std::vector<Region> region;  // per object
  std::vector<std::string> name;
  std::vector<std::vector<Ev>> prog;  // per wave
  int obj(const std::string& n, long lo, long hi) {
    region.push_back({lo, hi});
    name.push_back(n);
    return static_cast<int>(region.size()) - 1;
  }
};

static bool overlap(const Region& a, const Region& b) { return a.lo < b.hi && b.lo < a.hi; }

// Replays the programs; returns an empty string or the first violation.
static std::string check(const Model& m) {
  const int W = static_cast<int>(m.prog.size());
  const int NO = static_cast<int>(m.region.size());
  const int INF = 1 << 30;
  // done[w][o]: epoch in which wave w's share of o's DMA was waited for (INF: never);
  // issued[w][o]: epoch of issue (-1: this wave issues none of it)
  std::vector<std::vector<int>> done(W, std::vector<int>(NO, INF)), issued(W, std::vector<int>(NO, -1));
  std::vector<std::vector<int>> reads(NO);  // epochs of all reads
  std::vector<int> barriers(W, 0);
  std::vector<int> stored(NO, -1);        // last epoch a wave stored the object (WRITE), -1: never
  std::vector<int> first_store(NO, 1 << 30);
  for (int w = 0; w < W; ++w) {
    int e = 0;
    for (const Ev& ev : m.prog[w]) {
      if (ev.kind == BARRIER) ++e;
      if (ev.kind == WRITE) {
        stored[ev.obj] = std::max(stored[ev.obj], e);
        first_store[ev.obj] = std::min(first_store[ev.obj], e);
      }
    }
  }
  struct Write { int w, obj, epoch; bool dma; };
  std::vector<Write> writes;
  for (int w = 0; w < W; ++w) {
    int e = 0;
    std::vector<std::pair<int, int>> queue;  // (obj, instructions) outstanding, issue order
    for (const Ev& ev : m.prog[w]) {
      switch (ev.kind) {
        case ISSUE:
          if (ev.count > 0) {
            queue.push_back({ev.obj, ev.count});
            issued[w][ev.obj] = e;
          }
          writes.push_back({w, ev.obj, e, true});
          break;
        case WAIT_LEAVE: {
          int out = 0;
          for (auto& q : queue) out += q.second;
          while (out > ev.count && !queue.empty()) {
            const int take = std::min(queue.front().second, out - ev.count);
            queue.front().second -= take;
            out -= take;
            if (queue.front().second == 0) {
              done[w][queue.front().first] = e;
              queue.erase(queue.begin());
            }
          }
          break;
        }
        case BARRIER: ++e; ++barriers[w]; break;
        case READ: reads[ev.obj].push_back(e); break;
        case WRITE: writes.push_back({w, ev.obj, e, false}); break;
      }
      if (ev.kind == READ && stored[ev.obj] >= 0) {  // stored by waves: a barrier must follow every store
        if (!(stored[ev.obj] < e))
          return "wave " + std::to_string(w) + " reads " + m.name[ev.obj] + " in epoch " + std::to_string(e) +
                 " before every wave's store of it is published";
      } else if (ev.kind == READ) {
        for (int v = 0; v < W; ++v)
          if (issued[v][ev.obj] >= 0 && !(done[v][ev.obj] < e))
            return "wave " + std::to_string(w) + " reads " + m.name[ev.obj] + " in epoch " + std::to_string(e) +
                   " before wave " + std::to_string(v) + "'s DMA of it was waited for and published";
        bool any = false;
        for (int v = 0; v < W; ++v) any |= issued[v][ev.obj] >= 0;
        if (!any) return "wave " + std::to_string(w) + " reads " + m.name[ev.obj] + ", which no wave loads";
      }
    }
    if (!queue.empty()) return "wave " + std::to_string(w) + " exits with " + m.name[queue.front().first] + " in flight";
  }
  for (int w = 1; w < W; ++w)
    if (barriers[w] != barriers[0]) return "waves pass different numbers of barriers";
  // write-after-read and write-after-DMA on overlapping regions: the earlier occupant
  // is every object with a read or an issue strictly before the write's epoch
  for (const Write& wr : writes) {
    for (int o = 0; o < NO; ++o) {
      if (o == wr.obj || !overlap(m.region[o], m.region[wr.obj])) continue;
      int first_issue = first_store[o];  // an object stored by the waves is present from its first store
      for (int v = 0; v < W; ++v)
        if (issued[v][o] >= 0) first_issue = std::min(first_issue, issued[v][o]);
      if (first_issue > wr.epoch) continue;  // a later occupant
      if (!wr.dma && first_issue == wr.epoch) continue;  // stores of one epoch to distinct objects
      if (wr.dma && first_issue == wr.epoch) {
        // two DMAs into overlapping regions issued in the same epoch
        if (o < wr.obj) return m.name[wr.obj] + " and " + m.name[o] + " are loaded into overlapping LDS in one epoch";
        continue;
      }
      for (int r : reads[o])
        if (r >= wr.epoch)
          return std::string(wr.dma ? "DMA of " : "output staging ") + m.name[wr.obj] + " (wave " +
                 std::to_string(wr.w) + ", epoch " + std::to_string(wr.epoch) + ") overwrites " + m.name[o] +
                 " still read in epoch " + std::to_string(r);
      for (int v = 0; v < W; ++v)
        if (issued[v][o] >= 0 && !(done[v][o] < wr.epoch))
          return std::string(wr.dma ? "DMA of " : "output staging ") + m.name[wr.obj] +
                 " overwrites " + m.name[o] + " whose DMA may still land";
    }
  }
  return "";
}

// ---- the pipelined kernel (attn_fwd_bf16_pipe<D, W, rope, false>; rotating Q on load
// adds no LDS traffic: the angles are computed in registers)
template <int D>
static std::string pipe_case(int W, int kend) {
  using G = Geometry<D>;
  const int BM = 32 * W, BN = G::kBlockN, SK = G::kStepKeys, S = G::kStages;
  const long SE = G::kStageElems, KE = G::kKElems;
  const int ntiles = (kend + BN - 1) / BN, nsteps = (kend + SK - 1) / SK;
  Model m;
  const int q = m.obj("Q", pipe_q_elem<D>(), pipe_q_elem<D>() + G::q_pad_elems(BM));
  if (pipe_q_elem<D>() + G::q_pad_elems(BM) > pipe_lds_elems<D>(BM)) return "Q tile outside the LDS";
  std::vector<int> K(ntiles), V(ntiles);
  for (int t = 0; t < ntiles; ++t) {
    K[t] = m.obj("K" + std::to_string(t), (t % S) * SE, (t % S) * SE + KE);
    V[t] = m.obj("V" + std::to_string(t), (t % S) * SE + KE, (t % S + 1) * SE);
  }
  std::vector<int> O(W);
  for (int w = 0; w < W; ++w) O[w] = m.obj("O" + std::to_string(w), w * 32L * (D + 8), (w + 1) * 32L * (D + 8));
  m.prog.resize(W);
  for (int w = 0; w < W; ++w) {
    auto& p = m.prog[w];
    const int kd = G::k_dma_of(w, W), vd = G::v_dma_of(w, W);
    auto issue_tile = [&](int t) {
      p.push_back({ISSUE, K[t], kd});
      p.push_back({ISSUE, V[t], vd});
    };
    p.push_back({ISSUE, q, G::q_pad_dma_of(w, W, BM)});
    issue_tile(0);
    const bool early1 = kPipePrologueTiles >= 2;
    if (ntiles > 1 && early1) issue_tile(1);
    // wait for Q and K of tile 0 (V of tile 0 and, if issued, tile 1 stay in flight)
    const bool old_count = mutated("pipe_prologue_old_count");  // a count still leaving tile 1 out
    const int left = vd + (ntiles > 1 && (early1 || old_count) ? kd + vd : 0);
    p.push_back({WAIT_LEAVE, -1, left + (mutated("pipe_prologue_short") ? 1 : 0)});
    p.push_back({BARRIER, -1, 0});
    if (ntiles > 1 && !early1) issue_tile(1);  // tile 1 right after the first barrier
    p.push_back({READ, q, 0});
    p.push_back({READ, K[0], 0});  // QK of step 0
    if (nsteps > 1) p.push_back({READ, K[pipe_k_step(0) * SK / BN], 0});
    for (int j = 1; j <= nsteps; ++j) {
      if (pipe_syncs(j) != mutated("pipe_sync_even")) {
        p.push_back({WAIT_LEAVE, -1, 0});
        const int tn = pipe_issue_tile(j) + (mutated("pipe_issue_early") ? 1 : 0);
        if (mutated("pipe_issue_before_barrier") && tn < ntiles) issue_tile(tn);
        p.push_back({BARRIER, -1, 0});
        if (!mutated("pipe_issue_before_barrier") && tn < ntiles) issue_tile(tn);
      }
      if (j + 1 < nsteps) p.push_back({READ, K[pipe_k_step(j) * SK / BN], 0});
      p.push_back({READ, V[pipe_v_step(j) * SK / BN], 0});
    }
    if (!mutated("pipe_no_final_barrier")) p.push_back({BARRIER, -1, 0});
    p.push_back({WRITE, O[w], 0});
  }
  return check(m);
}

// ---- the key-split pipelined kernel (attn_fwd_bf16_pipe<D, W, rope, NG>): NG wave
// groups of W/NG waves, each wave one step (1/NG of a tile) per iteration; K and V rings
template <int D>
static std::string split_case(int W, int kend, int NG = 2) {
  using G = SplitGeometry<D>;
  const int QB = W / NG, BM = 32 * QB, BN = G::kBlockN;
  const long KE = G::kKElems, VE = G::kVElems, OP = D + 8;
  const int ntiles = (kend + BN - 1) / BN, nsteps = ntiles;
  Model m;
  const int q = m.obj("Q", G::kQElem, G::kQElem + G::q_pad_elems(BM));
  if (G::kQElem + G::q_pad_elems(BM) > G::lds_elems(BM) || G::lds_elems(BM) * 2 > 160 * 1024)
    return "Q tile outside the LDS";
  std::vector<int> K(ntiles), V(ntiles);
  for (int t = 0; t < ntiles; ++t) {
    K[t] = m.obj("K" + std::to_string(t), G::k_slot_elem(t), G::k_slot_elem(t) + KE);
    V[t] = m.obj("V" + std::to_string(t), G::v_slot_elem(t), G::v_slot_elem(t) + VE);
  }
  // group 0's output staging rows, then the other groups' partial results (13 x 64 x 16
  // bytes per wave), partial (g - 1) * QB + b for group g, query block b
  std::vector<int> O(QB), P((NG - 1) * QB);
  const long part0 = QB * 32L * OP, part_elems = 13L * 64 * 8;
  for (int b = 0; b < QB; ++b) O[b] = m.obj("O" + std::to_string(b), b * 32L * OP, (b + 1) * 32L * OP);
  for (int i = 0; i < (NG - 1) * QB; ++i)
    P[i] = m.obj("partial" + std::to_string(i), part0 + i * part_elems, part0 + (i + 1) * part_elems);
  if (part0 + (NG - 1) * QB * part_elems > G::lds_elems(BM)) return "merge buffers outside the LDS";
  m.prog.resize(W);
  for (int w = 0; w < W; ++w) {
    auto& p = m.prog[w];
    const int grp = w / QB, qb = w % QB;
    const int kd = G::k_dma_of(w, W), vd = G::v_dma_of(w, W);
    p.push_back({ISSUE, q, G::q_pad_dma_of(w, W, BM)});
    p.push_back({ISSUE, K[0], kd});
    if (ntiles > 1) p.push_back({ISSUE, K[1], kd});
    p.push_back({ISSUE, V[0], vd});
    p.push_back({WAIT_LEAVE, -1, vd + (ntiles > 1 ? kd : 0)});
    p.push_back({BARRIER, -1, 0});
    p.push_back({READ, q, 0});
    p.push_back({READ, K[0], 0});  // QK of step 0
    for (int j = 0; j <= nsteps; ++j) {
      p.push_back({WAIT_LEAVE, -1, (j < ntiles ? vd : 0) + (mutated("split_leave_k") ? kd : 0)});
      p.push_back({BARRIER, -1, 0});
      const int tk = split_issue_k(j) + (mutated("split_k_early") ? 1 : 0), tv = split_issue_v(j);
      if (tk < ntiles) p.push_back({ISSUE, K[tk], kd});
      if (tv < ntiles) p.push_back({ISSUE, V[tv], vd});
      if (j + 1 < nsteps) p.push_back({READ, K[split_k_tile(j)], 0});
      if (j >= 1) p.push_back({READ, V[split_v_tile(j)], 0});
    }
    p.push_back({BARRIER, -1, 0});
    if (grp > 0) p.push_back({WRITE, P[(grp - 1) * QB + qb], 0});
    if (!mutated("split_merge_no_barrier")) p.push_back({BARRIER, -1, 0});
    if (grp == 0) {
      for (int g = 1; g < NG; ++g) p.push_back({READ, P[(g - 1) * QB + qb], 0});
      p.push_back({WRITE, O[qb], 0});
    }
    if (mutated("split_merge_no_barrier")) p.push_back({BARRIER, -1, 0});
  }
  return check(m);
}

// ---- the phased kernel (attn_fwd_bf16<D, *>, 8 waves in two groups)
template <int D>
static std::string phased_case(int kend) {
  using G = Geometry<D>;
  const int W = 8, BM = 256, BN = G::kBlockN, SK = G::kStepKeys, S = G::kStages, N = G::kStepsPerTile;
  const long SE = G::kStageElems, KE = G::kKElems;
  const int ntiles = (kend + BN - 1) / BN, nsteps = (kend + SK - 1) / SK;
  const int QDMA_W = G::q_dma(BM) / W;
  Model m;
  const int qa = m.obj("Q rows 0-127", (S - 1) * SE, (S - 1) * SE + 128L * D);
  const int qb = m.obj("Q rows 128-255", (S - 1) * SE + 128L * D, (S - 1) * SE + 256L * D);
  std::vector<int> K(ntiles), V(ntiles);
  for (int t = 0; t < ntiles; ++t) {
    K[t] = m.obj("K" + std::to_string(t), (t % S) * SE, (t % S) * SE + KE);
    V[t] = m.obj("V" + std::to_string(t), (t % S) * SE + KE, (t % S + 1) * SE);
  }
  std::vector<int> O(W);
  for (int w = 0; w < W; ++w) O[w] = m.obj("O" + std::to_string(w), w * 32L * (D + 8), (w + 1) * 32L * (D + 8));
  auto tile_of = [&](int step) { return step * SK / BN; };
  m.prog.resize(W);
  for (int w = 0; w < W; ++w) {
    auto& p = m.prog[w];
    const int kd = G::k_dma_of(w, W), vd = G::v_dma_of(w, W);
    int t_issue = 1, t_wait = 1, v_pending = -1;
    auto issue_phase = [&](int t) {
      return phased_issue_phase(t, N, S) - (mutated("phased_issue_early") && t >= S ? 2 : 0);
    };
    auto wait_phase = [&](int t) { return phased_wait_phase(t, N) + (mutated("phased_wait_late") ? 2 : 0); };
    auto stage_begin = [&](int ph) {
      if (v_pending >= 0) {
        p.push_back({ISSUE, V[v_pending], vd});
        v_pending = -1;
      }
      if (t_issue < ntiles && issue_phase(t_issue) == ph) {
        p.push_back({ISSUE, K[t_issue], kd});
        if (S >= 3) v_pending = t_issue;
        else p.push_back({ISSUE, V[t_issue], vd});
        ++t_issue;
      }
    };
    auto stage_end = [&](int ph) {
      if (ph == 0) p.push_back({WAIT_LEAVE, -1, S >= 3 && t_issue >= 2 ? kd : 0});
      if (t_wait < ntiles && wait_phase(t_wait) == ph) {
        p.push_back({WAIT_LEAVE, -1, 0});
        ++t_wait;
      }
    };
    auto phase = [&](int ph, const std::vector<int>& rd) {
      stage_begin(ph);
      for (int o : rd) p.push_back({READ, o, 0});
      stage_end(ph);
      p.push_back({BARRIER, -1, 0});
    };
    // prologue
    p.push_back({ISSUE, qa, QDMA_W / 2});
    p.push_back({ISSUE, K[0], kd});
    p.push_back({ISSUE, qb, QDMA_W - QDMA_W / 2});
    p.push_back({ISSUE, V[0], vd});
    p.push_back({WAIT_LEAVE, -1, QDMA_W / 2 + G::kVDma / W});
    p.push_back({BARRIER, -1, 0});
    const bool lead = w < W / 2;
    const int qmine = lead ? qa : qb;
    // slot list of this wave: slot 0 = MFMA(0), then VALU(j), MFMA(j+1)
    std::vector<std::vector<int>> slots;
    slots.push_back({qmine, K[0]});
    for (int j = 0; j < nsteps; ++j) {
      std::vector<int> valu;
      if (j + 1 < nsteps) valu.push_back(K[tile_of(j + 1)]);
      slots.push_back(valu);
      std::vector<int> mfma;
      if (D == 128 && j + 1 < nsteps) mfma.push_back(K[tile_of(j + 1)]);  // the rest of K (head_dim 128)
      mfma.push_back(V[tile_of(j)]);
      slots.push_back(mfma);
    }
    int ph = 0;
    if (!lead) phase(ph++, {});
    for (const auto& s : slots) phase(ph++, s);
    if (lead) phase(ph++, {});
    // epilogue: the wave's output rows staged in the dead K/V stages
    p.push_back({WRITE, O[w], 0});
  }
  return check(m);
}

int main(int argc, char** argv) {
  if (argc > 1) g_mutation = argv[1];
  std::vector<int> kends;
  for (int k = 1; k <= 1100; ++k) kends.push_back(k);
  for (int k : {1536, 2048, 2049, 4095, 4096, 10752, 12288}) kends.push_back(k);
  long cases = 0;
  for (int kend : kends) {
    std::string r;
    const char* what = "";
    if ((r = pipe_case<96>(8, kend)).size()) what = "pipe<96, 8>";
    else if ((r = pipe_case<96>(4, kend)).size()) what = "pipe<96, 4>";
    else if ((r = split_case<96>(8, kend)).size()) what = "pipe<96, 8, split>";
    else if ((r = split_case<96>(8, kend, 4)).size()) what = "pipe<96, 8, four groups>";
    else if ((r = phased_case<64>(kend)).size()) what = "phased<64>";
    else if ((r = phased_case<96>(kend)).size()) what = "phased<96>";
    else if ((r = phased_case<128>(kend)).size()) what = "phased<128>";
    if (r.size()) {
      printf("violation: %s, %d keys: %s\n", what, kend, r.c_str());
      return 1;
    }
    cases += 7;
  }
  printf("ok %ld\n", cases);
  return 0;
}
