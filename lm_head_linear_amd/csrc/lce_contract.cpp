// lce_contract.cpp -- host-only contract of liblce.so: status names, the two
// budgets, the peak-cell reporter and workspace planning.  Integer arithmetic
// only; nothing here touches a device.
//
// Source: "Loss functions and resident-context kernels" (algenta docs), the
// lossk function table, "Status codes" and "The two budgets are genuinely
// different questions".
#include <cmath>
#include <mutex>

#include "lce_internal.h"

namespace lce {

bool finite_scalar(double x) { return std::isfinite(x); }

size_t dtype_size(int32_t dtype) {
  switch (dtype) {
    case LCE_BF16: return 2;
    case LCE_F16: return 2;
    case LCE_F32: return 4;
    case LCE_F64: return 8;
    case LCE_I64: return 8;
    case LCE_U8: return 1;
    default: return 0;
  }
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

namespace {

struct SlabChoice {
  int64_t slab = 0, slab0 = 0, splits = 1;
  double us = 0.0;   // modelled backward time
};

// Modelled time of one slab-pipeline launch: d_hidden (split `sp` ways) and
// d_weight of `prev` rows with the logit gradient of `next` rows, packed.
double launch_us(int64_t n, int64_t D, int64_t prev, int64_t next, int64_t sp, int64_t td,
                 int64_t tn, int64_t out_tiles) {
  const int64_t nt[3] = {prev > 0 ? out_tiles * sp : 0, prev > 0 ? ceil_div(prev, 256) * td : 0,
                         next > 0 ? ceil_div(next, 256) * tn : 0};
  const double dur[3] = {tile_us_dhidden(round_up(ceil_div(prev > 0 ? prev : 1, sp), 64)),
                         tile_us_dweight(n), tile_us_dlogit(D)};
  PackCounts pc;
  int slots = 0;
  double ms = 0.0;
  if (!pack_tiles(nt, dur, &pc, &slots, &ms)) {
    // hardware dispatch in product order: work spread over the compute
    // units, plus a tail of about one tile
    double work = 0.0, longest = 0.0;
    for (int j = 0; j < 3; ++j) {
      work += double(nt[j]) * (dur[j] + 1.0);
      if (nt[j] > 0 && dur[j] > longest) longest = dur[j];
    }
    ms = work / kComputeUnits + longest;
  }
  return ms + kLaunchUs;
}

// The slab (a multiple of 256 rows, at most s_max), the first slab and the
// d_hidden split count with the least modelled backward time, among the
// choices whose launches hold at most three tiles per compute unit (coarser
// work is where in-order dispatch leaves a long tail and packing pays); slab
// 0 when there is none.  The search is memoized per shape.
SlabChoice choose_slabs(int64_t n, int64_t D, int64_t V, int64_t s_max, int64_t tn, int64_t td,
                        int64_t out_tiles) {
  struct Entry {
    int64_t key[4];
    SlabChoice c;
  };
  static std::mutex mu;
  static Entry memo[32];
  static int n_memo = 0, next_slot = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_memo; ++i)
      if (memo[i].key[0] == n && memo[i].key[1] == D && memo[i].key[2] == V &&
          memo[i].key[3] == s_max)
        return memo[i].c;
  }
  SlabChoice best;
  const int64_t s_min = s_max - 8 * 256 > 256 ? s_max - 8 * 256 : 256;
  for (int64_t S = s_max; S >= s_min; S -= 256) {
    // slab 0: the rows of one round of compute units, or a whole slab
    int64_t firsts[2] = {S, S};
    if (tn <= kComputeUnits) {
      const int64_t r0 = (kComputeUnits / tn) * 256;
      if (r0 < S) firsts[1] = r0;
    }
    for (int f = 0; f < 2; ++f) {
      if (f == 1 && firsts[1] == firsts[0]) continue;
      const int64_t s0 = firsts[f] < V ? firsts[f] : V;
      // slab rows: s0, then S ..., then the remainder
      const int64_t ns = V > s0 ? 1 + ceil_div(V - s0, S) : 1;
      const int64_t last = ns > 1 ? V - s0 - (ns - 2) * S : s0;
      for (int64_t sp = 1; sp <= 16; sp *= 2) {
        if (sp > 1 && S / sp < 512) break;
        const int64_t busiest = out_tiles * sp + ceil_div(S, 256) * (td + tn);
        if (busiest > 3 * kComputeUnits) continue;
        double t = launch_us(n, D, 0, s0, sp, td, tn, out_tiles);
        if (ns == 1) {
          t += launch_us(n, D, s0, 0, sp, td, tn, out_tiles);
        } else {
          t += launch_us(n, D, s0, ns > 2 ? S : last, sp, td, tn, out_tiles);
          if (ns > 3) t += double(ns - 3) * launch_us(n, D, S, S, sp, td, tn, out_tiles);
          if (ns > 2) t += launch_us(n, D, S, last, sp, td, tn, out_tiles);
          t += launch_us(n, D, last, 0, sp, td, tn, out_tiles);
        }
        if (best.slab == 0 || t < best.us) {
          best.slab = S;
          best.slab0 = s0;
          best.splits = sp;
          best.us = t;
        }
      }
    }
  }
  std::lock_guard<std::mutex> lock(mu);
  Entry &e = memo[next_slot];
  next_slot = (next_slot + 1) % 32;
  if (n_memo < 32) ++n_memo;
  e.key[0] = n; e.key[1] = D; e.key[2] = V; e.key[3] = s_max;
  e.c = best;
  return best;
}

}  // namespace

int32_t plan_ce(int64_t n, int64_t D, int64_t V, int64_t chunk, int32_t dtype, CEPlan *p) {
  int32_t st = lce_dims_check(n, D, V);
  if (st != LCE_OK) return st;
  st = lce_chunk_check(chunk, V);
  if (st != LCE_OK) return st;
  if (dtype != LCE_BF16 && dtype != LCE_F16 && dtype != LCE_F64) return LCE_DTYPE_MISMATCH;

  CEPlan q;
  q.dtype = dtype;
  q.n = n; q.D = D; q.V = V; q.chunk = chunk;
  const bool bf = dtype != LCE_F64;   // 16-bit inputs (bf16 or fp16)
  q.elem = bf ? 2 : 8;
  q.acc = bf ? 4 : 8;
  const int64_t tile_m = bf ? kBf16TileM : kF64TileM;
  const int64_t budget = chunk * V;  // logit-derived cells allowed at once (<= 2^27)

  // Forward: each token keeps n_vparts (max, sum) pairs; as many tokens run
  // per launch as fit the chunk*vocab cell budget.
  q.wave_m = bf ? kBf16WaveM : kF64WaveM;
  q.n_vparts = ceil_div(V, q.wave_m);
  int64_t tpp = budget / (2 * q.n_vparts);
  if (tpp < 1) tpp = 1;
  q.tok_per_pass = tpp < n ? tpp : n;

  // Backward: the logit-gradient buffer holds a slab of vocabulary rows for
  // every token, at most chunk*vocab cells.
  q.d_ld = round_up(n, 64);
  int64_t slab_max = budget / q.d_ld;
  const int64_t tile_n = bf ? 256 : 128;
  const int64_t out_tiles = ceil_div(n, tile_m) * ceil_div(D, tile_n);
  // Workgroups resident at once: one 16-bit tile per compute unit, two fp64
  // tiles (the fp64 core runs two workgroups per CU).
  const int64_t slots = bf ? kComputeUnits : kF64PerCu * kComputeUnits;
  // Split the vocabulary reduction of d_hidden so that the grid has about one
  // workgroup per slot, keeping each split at least 512 deep.
  auto dh_splits_for = [&](int64_t slab) {
    int64_t sp = ceil_div(slots, out_tiles);
    if (sp > slab / 512) sp = slab / 512;
    if (sp > 16) sp = 16;
    return sp < 1 ? int64_t(1) : sp;
  };
  if (slab_max >= tile_m) {
    // A launch costs about (rounds of tiles over the slots) x (depth +
    // epilogue).  Pick the slab (a multiple of the tile rows) with the lowest
    // modelled total over the three backward GEMMs of every slab; ties go to
    // the larger slab.
    slab_max = slab_max / tile_m * tile_m;
    if (slab_max > round_up(V, tile_m)) slab_max = round_up(V, tile_m);
    const int64_t tn = ceil_div(n, tile_m), td = ceil_div(D, tile_n);
    const int64_t kEpi = 256, kLaunch = 64;
    auto rounds = [&](int64_t wgs) { return ceil_div(wgs, slots); };
    auto slab_cost = [&](int64_t rows, int64_t sp) {
      const int64_t tm = ceil_div(rows, tile_m);
      return rounds(tm * tn) * (D + kEpi) + rounds(tm * td) * (n + kEpi) +
             rounds(out_tiles * sp) * (ceil_div(rows, sp) + kEpi) + 3 * kLaunch;
    };
    int64_t best = -1, best_cost = 0;
    for (int64_t S = tile_m; S <= slab_max; S += tile_m) {
      const int64_t ns = ceil_div(V, S);
      const int64_t sp = dh_splits_for(S);
      const int64_t c = (ns - 1) * slab_cost(S, sp) + slab_cost(V - (ns - 1) * S, sp);
      if (best < 0 || c <= best_cost) { best = S; best_cost = c; }
    }
    q.slab = best < V ? best : V;
    q.n_slabs = ceil_div(V, q.slab);
  } else {
    if (slab_max >= 32) slab_max = slab_max / 32 * 32;
    if (slab_max < 1) slab_max = 1;
    if (slab_max >= V) {
      q.slab = V;
      q.n_slabs = 1;
    } else {  // balanced slabs
      q.n_slabs = ceil_div(V, slab_max);
      int64_t gran = slab_max >= tile_m ? tile_m : (slab_max >= 32 ? 32 : 1);
      int64_t bal = round_up(ceil_div(V, q.n_slabs), gran);
      q.slab = bal <= slab_max ? bal : slab_max;
      q.n_slabs = ceil_div(V, q.slab);
    }
  }
  q.dh_splits = dh_splits_for(q.slab);

  // bf16 slab pipeline: two buffers of pslab rows, 2 * pslab * d_ld <= budget.
  // The slab is the largest multiple of 256 rows the budget allows (measured:
  // fewer, larger launches win; each launch pays fixed prologue/epilogue tails
  // and one d_hidden read-modify-write).  The d_hidden split count comes from
  // a model of each launch as max(total workgroup work / CUs, longest
  // workgroup) with work = depth (x 1.25 for the MN-major d_hidden operands)
  // + epilogue.
  if (bf) {
    const int64_t half = budget / (2 * q.d_ld) / tile_m * tile_m;
    const int64_t tn = ceil_div(n, tile_m), td = ceil_div(D, tile_n);
    const int64_t kEpi = 256, kLaunch = 64;
    auto launch_cost = [&](int64_t prev_rows, int64_t next_rows, int64_t sp) {
      int64_t work = 0, longest = 0;
      if (prev_rows > 0) {
        const int64_t tm = ceil_div(prev_rows, tile_m);
        const int64_t dh_wg = (ceil_div(prev_rows, sp) * 5) / 4 + kEpi;
        work += out_tiles * sp * dh_wg + tm * td * (n + kEpi);
        longest = dh_wg > n + kEpi ? dh_wg : n + kEpi;
      }
      if (next_rows > 0) {
        const int64_t tm = ceil_div(next_rows, tile_m);
        work += tm * tn * (D + kEpi);
        if (D + kEpi > longest) longest = D + kEpi;
      }
      const int64_t spread = ceil_div(work, kComputeUnits);
      return (spread > longest ? spread : longest) + kLaunch;
    };
    const int64_t S = half < round_up(V, tile_m) ? half : round_up(V, tile_m);
    if (S >= tile_m) {
      const int64_t ns = ceil_div(V, S);
      const int64_t last = V - (ns - 1) * S;
      int64_t best_sp = 1, best_cost = -1;
      for (int64_t sp = 1; sp <= 16; sp *= 2) {
        if (sp > 1 && S / sp < 512) break;
        // launches: (-, 0), (0, 1), ..., (ns-2, ns-1), (ns-1, -)
        int64_t c = launch_cost(0, ns == 1 ? last : S, sp);
        if (ns >= 3) c += (ns - 2) * launch_cost(S, S, sp);
        if (ns >= 2) c += launch_cost(S, last, sp);
        c += launch_cost(last, 0, sp);
        if (best_cost < 0 || c < best_cost) {
          best_sp = sp;
          best_cost = c;
        }
      }
      // forward (rounds of vocabulary x token tiles, each D deep) + backward,
      // for the single call's choice below
      q.model_two = ceil_div(ceil_div(V, tile_m) * tn * (D + kEpi), kComputeUnits) + kLaunch +
                    best_cost;
      // The launches themselves are packed onto the compute units
      // (pack_tiles), so the slab, its d_hidden split count and the first
      // slab are chosen by the packed makespans of all launches of the
      // backward (choose_slabs).
      const SlabChoice c = choose_slabs(n, D, V, S, tn, td, out_tiles);
      if (c.slab > 0) {
        q.pslab = c.slab;
        q.pslab0 = c.slab0;
        q.pdh_splits = c.splits;
        q.ppacked = true;
        q.model_bwd_us = c.us;
      } else {
        // Finer-grained launches (more than three tiles per compute unit):
        // hardware dispatch balances them; the largest slab, the split count
        // of the launch model above and a first slab of one round.
        q.pslab = S < V ? S : V;
        q.pdh_splits = best_sp;
        q.pslab0 = q.pslab;
        if (tn <= kComputeUnits) {
          const int64_t r0 = (kComputeUnits / tn) * tile_m;
          if (r0 < q.pslab && ceil_div(q.pslab, tile_m) * tn > kComputeUnits) q.pslab0 = r0;
        }
      }
      q.pn_slabs = V > q.pslab0 ? 1 + ceil_div(V - q.pslab0, q.pslab) : 1;
    }
  }

  // Workspace: [control | forward partials | zy | per-token loss] and the
  // backward's [slab buffer | d_hidden split accumulators] overlap the
  // forward region (the two calls never run on one workspace at once).
  size_t off = kControlBytes;
  size_t fwd_begin = off;
  q.off_partials = off;
  off = align256(off + size_t(q.tok_per_pass) * size_t(q.n_vparts) * 2 * q.acc);
  q.off_zy = off;
  off = align256(off + size_t(n) * q.acc);
  q.off_losstok = off;
  off = align256(off + size_t(n) * 8);
  size_t fwd_end = off;
  off = fwd_begin;
  q.off_dbuf = off;
  {
    int64_t cells = q.slab * q.d_ld;
    if (2 * q.pslab * q.d_ld > cells) cells = 2 * q.pslab * q.d_ld;
    off = align256(off + size_t(cells) * q.elem);
  }
  q.off_dhacc = off;
  {
    const int64_t sp = q.dh_splits > q.pdh_splits ? q.dh_splits : q.pdh_splits;
    off = align256(off + size_t(sp) * size_t(n) * size_t(D) * q.acc);
  }
  q.off_ht = off;
  off = align256(off + size_t(D) * size_t(q.d_ld) * q.elem);
  q.off_zyb = off;
  if (bf) off = align256(off + size_t(n) * q.acc);
  // shard-local target ids (vocabulary-shard calls), past both regions
  off = off > fwd_end ? off : fwd_end;
  q.off_yloc = off;
  q.total = align256(off + size_t(n) * sizeof(int64_t));

  // Single-call layout: the forward region, then the kept logits, the d_hidden
  // split accumulators and H^T, all live at once.  The logits take V * f_ld
  // cells (at most chunk*vocab); f_ld also covers, at two 16-bit values per
  // cell, the gradient rows zero-padded to a multiple of 64 tokens.
  //
  // Whether keeping pays is decided by the same launch model as the slab
  // pipeline (times in k-rows of one 256x256 tile on one compute unit,
  // about 28 ns each): the kept path saves the recompute but writes the
  // logits in fp32 from the forward GEMM (4 bytes per kept cell, half of it
  // hidden behind that GEMM's matrix work), then reads them back and writes
  // the 16-bit gradient in a streaming pass (6 bytes per cell; about 128 KB
  // per unit at the chip's streaming rate), and runs d_hidden as one launch
  // over the whole vocabulary.  The logits are kept when the model puts that
  // path at least 1% ahead of the two-call algorithm (measured on
  // 512 x 151936 heads, single call against the two calls on one box:
  // 1.21-1.26x at d_model 4096, 1.01-1.05x at 1024; 1.14-1.16x at 256 x 1024).
  q.f_total = q.total;
  if (bf) {
    int64_t fld = round_up(n, 4);
    if (2 * fld < round_up(n, 64)) fld = round_up(n, 64) / 2;
    int64_t sp = ceil_div(kComputeUnits, out_tiles);
    if (sp > V / 512) sp = V / 512;
    if (sp > 32) sp = 32;
    if (sp < 1) sp = 1;
    {
      const int64_t kEpi = 256, kLaunch = 64, kBytesPerUnit = 128000;
      const int64_t tn = ceil_div(n, tile_m), td = ceil_div(D, tile_n);
      const int64_t fwd = ceil_div(ceil_div(V, tile_m) * tn * (D + 2 * kEpi), kComputeUnits);
      const int64_t kept = V * fld * 6 / kBytesPerUnit + V * fld * 4 / (2 * kBytesPerUnit);
      const int64_t dh_wg = (ceil_div(V, sp) * 5) / 4 + kEpi;
      const int64_t work = out_tiles * sp * dh_wg + ceil_div(V, tile_m) * td * (n + kEpi);
      const int64_t spread = ceil_div(work, kComputeUnits);
      q.model_single = fwd + kept + (spread > dh_wg ? spread : dh_wg) + 3 * kLaunch;
    }
    // (without a slab pipeline to compare with, keeping always pays)
    const bool pays = q.model_two == 0 || q.model_single * 101 < q.model_two * 100;
    if (fld <= chunk && q.tok_per_pass >= n && pays) {
      q.f_ok = true;
      q.f_ld = fld;
      q.f_sp = sp;
      size_t o = fwd_end;
      q.off_fz = o;
      o = align256(o + size_t(V) * size_t(fld) * 4);
      q.off_fdh = o;
      o = align256(o + size_t(q.f_sp) * size_t(n) * size_t(D) * 4);
      q.off_fht = o;
      o = align256(o + size_t(D) * size_t(q.d_ld) * 2);
      q.off_fyloc = o;
      o = align256(o + size_t(n) * sizeof(int64_t));
      if (o > q.f_total) q.f_total = o;
    }
  }
  *p = q;
  return LCE_OK;
}

namespace {

constexpr int kSlotsPerXcd = kPackSlots / kPackXcds;

// Best-fit decreasing under makespan T: every tile goes to the slot whose
// load it leaves closest to T (a new slot only when none has room).  Tiles
// of one product are identical, so placing them one by one fills the
// fullest slot that still has room as far as it goes, then the next fullest:
// done here in bulk.  gap is the per-tile cost of starting another tile on a
// slot.
bool pack_under(const int64_t k[3], const double dur[3], const int order[3], double T,
                double gap, uint8_t c[kSlotsPerXcd][3], int *used) {
  double load[kSlotsPerXcd] = {};
  int open = 0;
  for (int s = 0; s < kSlotsPerXcd; ++s) c[s][0] = c[s][1] = c[s][2] = 0;
  for (int oi = 0; oi < 3; ++oi) {
    const int j = order[oi];
    const double d = dur[j] + gap;
    int64_t left = k[j];
    if (left > 0 && d > T) return false;
    while (left > 0) {
      // the fullest open slot with room for one more tile of this product
      int best = -1;
      for (int s = 0; s < open; ++s)
        if (load[s] + d <= T && c[s][j] < 255 && (best < 0 || load[s] > load[best])) best = s;
      if (best < 0) {
        if (open == kSlotsPerXcd) return false;
        best = open++;
      }
      int64_t fit = int64_t((T - load[best]) / d);
      if (fit > 255 - c[best][j]) fit = 255 - c[best][j];
      if (fit > left) fit = left;
      if (fit < 1) return false;
      load[best] += double(fit) * d;
      c[best][j] = uint8_t(c[best][j] + fit);
      left -= fit;
    }
  }
  *used = open;
  return true;
}

// One XCD's share: the smallest makespan (to 0.5%) best-fit decreasing
// reaches; false when no makespan fits (a slot would need more than 255
// tiles of one product).
bool pack_xcd(const int64_t k[3], const double dur[3], uint8_t c[kSlotsPerXcd][3], int *used) {
  const double gap = 1.0;
  int order[3] = {0, 1, 2};
  for (int a = 0; a < 3; ++a)   // longest tiles first
    for (int b = a + 1; b < 3; ++b)
      if (dur[order[b]] > dur[order[a]]) {
        const int t = order[a];
        order[a] = order[b];
        order[b] = t;
      }
  double total = 0.0, longest = 0.0;
  for (int j = 0; j < 3; ++j) {
    total += double(k[j]) * (dur[j] + gap);
    if (k[j] > 0 && dur[j] + gap > longest) longest = dur[j] + gap;
  }
  if (total == 0.0) {
    *used = 0;
    for (int s = 0; s < kSlotsPerXcd; ++s) c[s][0] = c[s][1] = c[s][2] = 0;
    return true;
  }
  double lo = total / kSlotsPerXcd > longest ? total / kSlotsPerXcd : longest;
  double hi = lo;
  uint8_t tmp[kSlotsPerXcd][3];
  int u = 0;
  while (!pack_under(k, dur, order, hi, gap, tmp, &u)) {
    hi *= 1.125;
    if (hi > 2.0 * total + longest) return false;   // counts beyond 255 per slot
  }
  for (int s = 0; s < kSlotsPerXcd; ++s)
    for (int j = 0; j < 3; ++j) c[s][j] = tmp[s][j];
  *used = u;
  for (int it = 0; it < 10 && hi - lo > 0.005 * lo; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (pack_under(k, dur, order, mid, gap, tmp, &u)) {
      hi = mid;
      for (int s = 0; s < kSlotsPerXcd; ++s)
        for (int j = 0; j < 3; ++j) c[s][j] = tmp[s][j];
      *used = u;
    } else {
      lo = mid;
    }
  }
  return true;
}

}  // namespace

bool pack_tiles(const int64_t n[3], const double dur[3], PackCounts *out, int *slots,
                double *makespan) {
  // XCDs with the same tile counts get the same packing
  int64_t seen[kPackXcds][3];
  uint8_t packed[kPackXcds][kSlotsPerXcd][3];
  int used[kPackXcds];
  int n_seen = 0, most = 0;
  for (int x = 0; x < kPackXcds; ++x) {
    int64_t k[3];
    for (int j = 0; j < 3; ++j) k[j] = n[j] / kPackXcds + (x < n[j] % kPackXcds ? 1 : 0);
    int m = -1;
    for (int i = 0; i < n_seen; ++i)
      if (seen[i][0] == k[0] && seen[i][1] == k[1] && seen[i][2] == k[2]) m = i;
    if (m < 0) {
      m = n_seen++;
      for (int j = 0; j < 3; ++j) seen[m][j] = k[j];
      if (!pack_xcd(k, dur, packed[m], &used[m])) return false;
    }
    for (int s = 0; s < kSlotsPerXcd; ++s)
      for (int j = 0; j < 3; ++j) out->c[kPackXcds * s + x][j] = packed[m][s][j];
    if (used[m] > most) most = used[m];
  }
  *slots = most;
  if (makespan) {
    double worst = 0.0;
    for (int b = 0; b < kPackSlots; ++b) {
      double load = 0.0;
      for (int j = 0; j < 3; ++j) load += double(out->c[b][j]) * (dur[j] + 1.0);
      if (load > worst) worst = load;
    }
    *makespan = worst;
  }
  return true;
}

int32_t plan_distill(int64_t n, int64_t V, DistillPlan *p) {
  if (n < 1 || V < 1) return LCE_EMPTY_DIMENSION;
  if (n > LCE_MAX_N_TOK || V > LCE_MAX_VOCAB) return LCE_DIMENSION_TOO_LARGE;
  DistillPlan q;
  q.n = n; q.V = V;
  q.off_rows = kControlBytes;
  q.total = align256(q.off_rows + size_t(n) * 2 * sizeof(double));
  *p = q;
  return LCE_OK;
}

}  // namespace lce

using namespace lce;

extern "C" {

const char *lce_status_name(int32_t code) {
  static const char *const names[] = {
      "ok", "empty_dimension", "length_mismatch", "dimension_too_large",
      "work_budget_exceeded", "non_finite_scalar", "target_id_out_of_range",
      "chunk_exceeds_logit_budget", "unknown_objective", "device_error", "dtype_mismatch"};
  if (code < LCE_OK || code > LCE_DTYPE_MISMATCH) return "unknown_status";
  return names[code - LCE_OK];
}

int32_t lce_work_fits(int64_t n, int64_t d, int64_t v, int64_t ceiling) {
  if (n < 1 || d < 1 || v < 1 || ceiling < 0) return 0;
  // n*d*v <= ceiling  <=>  n <= floor(floor(ceiling / v) / d)
  const int64_t per_row = ceiling / v;
  return n <= per_row / d ? 1 : 0;
}

int32_t lce_dims_check(int64_t n_tok, int64_t d_model, int64_t vocab) {
  if (n_tok < 1 || d_model < 1 || vocab < 1) return LCE_EMPTY_DIMENSION;
  if (n_tok > LCE_MAX_N_TOK || d_model > LCE_MAX_D_MODEL || vocab > LCE_MAX_VOCAB)
    return LCE_DIMENSION_TOO_LARGE;
  return lce_work_fits(n_tok, d_model, vocab, LCE_MAX_WORK_CELLS) ? LCE_OK
                                                                  : LCE_WORK_BUDGET_EXCEEDED;
}

int32_t lce_chunk_check(int64_t chunk, int64_t vocab) {
  if (chunk < 1 || vocab < 1) return LCE_EMPTY_DIMENSION;
  // chunk*vocab > 2^27  <=>  chunk > floor(2^27 / vocab)
  return chunk > LCE_MAX_LOGIT_CELLS / vocab ? LCE_CHUNK_EXCEEDS_LOGIT_BUDGET : LCE_OK;
}

double lce_logit_cells(int64_t chunk, int64_t vocab) {
  if (chunk < 1 || vocab < 1) return -1.0;
  return double(chunk) * double(vocab);
}

int32_t lce_peak_cells(int64_t n_tok, int64_t vocab, int64_t chunk, lce_peak *out) {
  if (!out) return LCE_LENGTH_MISMATCH;
  if (n_tok < 1 || vocab < 1 || chunk < 1) {
    *out = lce_peak{-1.0, -1.0, -1.0, 0, LCE_EMPTY_DIMENSION};
    return LCE_EMPTY_DIMENSION;
  }
  const int64_t rows = chunk < n_tok ? chunk : n_tok;
  out->chunked_cells = lce_logit_cells(rows, vocab);
  out->materialized_cells = lce_logit_cells(n_tok, vocab);
  out->ratio = out->materialized_cells / out->chunked_cells;
  out->n_chunks = (n_tok + chunk - 1) / chunk;
  out->status = lce_chunk_check(chunk, vocab);
  return out->status;
}

int64_t lce_workspace_bytes(int64_t n_tok, int64_t d_model, int64_t vocab, int64_t chunk,
                            int32_t dtype) {
  CEPlan p;
  int32_t st = plan_ce(n_tok, d_model, vocab, chunk, dtype, &p);
  if (st != LCE_OK) return -int64_t(st);
  return int64_t(p.total) + 256;  // slack: the library aligns the base to 256 bytes
}

int64_t lce_forward_backward_workspace_bytes(int64_t n_tok, int64_t d_model, int64_t vocab,
                                             int64_t chunk, int32_t dtype) {
  CEPlan p;
  int32_t st = plan_ce(n_tok, d_model, vocab, chunk, dtype, &p);
  if (st != LCE_OK) return -int64_t(st);
  return int64_t(p.f_total) + 256;
}

int32_t lce_forward_backward_keeps_logits(int64_t n_tok, int64_t d_model, int64_t vocab,
                                          int64_t chunk, int32_t dtype) {
  CEPlan p;
  const int32_t st = plan_ce(n_tok, d_model, vocab, chunk, dtype, &p);
  if (st != LCE_OK) return -st;
  // the kept path reads every operand with the 16-byte pipelined core
  return p.f_ok && d_model % 64 == 0 ? 1 : 0;
}

int64_t lce_distill_workspace_bytes(int64_t n_tok, int64_t vocab) {
  DistillPlan p;
  int32_t st = plan_distill(n_tok, vocab, &p);
  if (st != LCE_OK) return -int64_t(st);
  return int64_t(p.total) + 256;
}

}  // extern "C"
