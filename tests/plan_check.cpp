// Host check of the CE planner (lce::plan_ce), built with g++ against
// lce_contract.cpp by tests/test_host_planner.py.
//
// Over a grid of token counts, model widths, vocabularies, chunks and input
// types it checks what every accepted plan promises:
//  * the logit-derived buffers stay within chunk * vocab cells: the
//    backward's slab buffer (rows x padded tokens; at least one vocabulary
//    row), the two buffers of the 16-bit slab pipeline, the single call's
//    kept logits, and the forward's per-block (max, sum) partials of the
//    tokens of one launch (at least one token);
//  * the slabs cover the vocabulary exactly (the pipeline's first slab, then
//    full slabs, then the remainder);
//  * split counts, strides and workspace offsets are sane: 256-byte aligned,
//    inside the reported workspace, regions live at the same time disjoint
//    (the single call's regions follow the forward region).
// Refusals must match the host checks (dims, chunk, dtype).
// Prints "ok <plans> <refused> <pipelined> <packed> <kept>" or the first
// failing case.
#include <cstdio>

#include "lce_internal.h"

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool fail(const char *what, int64_t n, int64_t D, int64_t V, int64_t c, int32_t dt) {
  std::printf("FAIL %s: n=%lld D=%lld V=%lld chunk=%lld dtype=%d\n", what, (long long)n,
              (long long)D, (long long)V, (long long)c, dt);
  return false;
}

struct Tally {
  int plans = 0, refused = 0, pipelined = 0, packed = 0, kept = 0;
};

bool check(int64_t n, int64_t D, int64_t V, int64_t chunk, int32_t dt, Tally *t) {
  lce::CEPlan p;
  const int32_t st = lce::plan_ce(n, D, V, chunk, dt, &p);
  int32_t want = lce_dims_check(n, D, V);
  if (want == LCE_OK) want = lce_chunk_check(chunk, V);
  if (want == LCE_OK && dt != LCE_BF16 && dt != LCE_F16 && dt != LCE_F64)
    want = LCE_DTYPE_MISMATCH;
  if (st != want) return fail("status differs from the host checks", n, D, V, chunk, dt);
  if (st != LCE_OK) {
    ++t->refused;
    return true;
  }
  ++t->plans;
  t->pipelined += p.pslab > 0;
  t->packed += p.ppacked;
  t->kept += p.f_ok;
  const bool bf = dt != LCE_F64;
  const int64_t budget = chunk * V;
  if (p.d_ld != ceil_div(n, 64) * 64) return fail("slab row stride", n, D, V, chunk, dt);
  // forward partials: two per block of wave_m vocabulary rows per token
  if (p.n_vparts != ceil_div(V, p.wave_m)) return fail("partials per token", n, D, V, chunk, dt);
  if (p.tok_per_pass < 1 || p.tok_per_pass > n) return fail("tokens per pass", n, D, V, chunk, dt);
  {
    const int64_t one = 2 * p.n_vparts;
    if (p.tok_per_pass * one > (budget > one ? budget : one))
      return fail("forward partials exceed chunk*vocab", n, D, V, chunk, dt);
  }
  // backward slab buffer (used when no pipeline is planned)
  if (p.slab < 1 || p.slab > V || p.n_slabs != ceil_div(V, p.slab))
    return fail("slabs do not cover the vocabulary", n, D, V, chunk, dt);
  if (p.slab * p.d_ld > (budget > p.d_ld ? budget : p.d_ld))
    return fail("slab buffer exceeds chunk*vocab", n, D, V, chunk, dt);
  if (p.dh_splits < 1 || p.dh_splits > 16) return fail("d_hidden splits", n, D, V, chunk, dt);
  if (p.pslab > 0) {
    if (!bf) return fail("slab pipeline planned for fp64", n, D, V, chunk, dt);
    if (2 * p.pslab * p.d_ld > budget)
      return fail("slab pipeline buffers exceed chunk*vocab", n, D, V, chunk, dt);
    if (p.pslab0 < 1 || p.pslab0 > p.pslab || (p.pslab < V && p.pslab % 256 != 0) ||
        p.pdh_splits < 1 || p.pdh_splits > 16)
      return fail("slab pipeline geometry", n, D, V, chunk, dt);
    // rows: pslab0, then pslab each, the last one short
    const int64_t covered = p.pslab0 + (p.pn_slabs - 1) * p.pslab;
    if (covered < V || (p.pn_slabs >= 2 && covered - p.pslab >= V))
      return fail("pipeline slabs do not cover the vocabulary", n, D, V, chunk, dt);
  }
  // workspace layout
  const size_t offs[] = {p.off_partials, p.off_zy,  p.off_losstok, p.off_dbuf,
                         p.off_dhacc,    p.off_ht,  p.off_zyb,     p.off_yloc};
  for (size_t o : offs)
    if (o % 256 != 0 || o < lce::kControlBytes || o >= p.total)
      return fail("workspace offset", n, D, V, chunk, dt);
  if (p.off_dhacc < p.off_dbuf + size_t(p.slab * p.d_ld) * p.elem ||
      p.off_ht < p.off_dhacc + size_t(p.dh_splits * n * D) * p.acc ||
      p.off_yloc < p.off_zy + size_t(n) * p.acc || p.total < p.off_yloc + size_t(n) * 8)
    return fail("workspace regions overlap", n, D, V, chunk, dt);
  if (p.pslab > 0 && p.off_dhacc < p.off_dbuf + size_t(2 * p.pslab * p.d_ld) * p.elem)
    return fail("pipeline buffers overlap the split accumulators", n, D, V, chunk, dt);
  // single call: kept logits [V][f_ld] fp32 when the whole batch fits a chunk
  if (p.f_total < p.total) return fail("single-call workspace", n, D, V, chunk, dt);
  if (p.f_ok) {
    if (!bf || p.f_ld < n || p.f_ld > chunk || 2 * p.f_ld < p.d_ld || p.tok_per_pass != n)
      return fail("kept-logit geometry", n, D, V, chunk, dt);
    if (V * p.f_ld > budget) return fail("kept logits exceed chunk*vocab", n, D, V, chunk, dt);
    const size_t fo[] = {p.off_fz, p.off_fdh, p.off_fht, p.off_fyloc};
    for (size_t o : fo)
      if (o % 256 != 0 || o >= p.f_total) return fail("single-call offset", n, D, V, chunk, dt);
    // (after the forward region; the two-call backward's regions are unused)
    if (p.off_fz < p.off_losstok + size_t(n) * 8 || p.off_fdh < p.off_fz + size_t(V * p.f_ld) * 4 ||
        p.off_fht < p.off_fdh + size_t(p.f_sp * n * D) * 4 ||
        p.off_fyloc < p.off_fht + size_t(D * p.d_ld) * 2 ||
        p.f_total < p.off_fyloc + size_t(n) * 8)
      return fail("single-call regions overlap", n, D, V, chunk, dt);
  }
  return true;
}

}  // namespace

int main() {
  const int64_t ns[] = {1, 3, 64, 100, 255, 256, 300, 517, 1000, 2048, 4097, 8192, 40000};
  const int64_t Ds[] = {1, 37, 64, 100, 256, 1024, 4096};
  const int64_t Vs[] = {1, 5, 33, 300, 1000, 3000, 40000, 128256, 151936, 262144};
  const int64_t chunks[] = {1, 2, 16, 64, 256, 300, 512, 883, 1024, 4096, 40000};
  const int32_t dts[] = {LCE_BF16, LCE_F16, LCE_F64, LCE_F32};
  Tally t;
  for (int64_t n : ns)
    for (int64_t D : Ds)
      for (int64_t V : Vs)
        for (int64_t c : chunks)
          for (int32_t dt : dts)
            if (!check(n, D, V, c, dt, &t)) return 1;
  // the chunk equal to the batch (the single call's case) and one past it
  for (int64_t n : ns)
    for (int64_t V : Vs)
      for (int64_t dc = 0; dc <= 1; ++dc)
        for (int32_t dt : dts)
          if (!check(n, 1024, V, n + dc, dt, &t)) return 1;
  std::printf("ok %d %d %d %d %d\n", t.plans, t.refused, t.pipelined, t.packed, t.kept);
  return 0;
}
