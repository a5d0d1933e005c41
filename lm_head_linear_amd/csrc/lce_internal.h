// lce_internal.h -- host-side pieces shared by the translation units of liblce.so.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/lce.h"

namespace lce {

// Device-side control block at offset 0 of every workspace.  The guard
// kernel fills bad/first_bad/count; the reduction kernels fill the sums.
struct Control {
  int32_t bad;          // nonzero when this call's target guard failed
  int32_t seen_bad;     // a guard failed in the last forward on this workspace
                        // or in a backward since (read by lce_loss_fetch)
  int64_t first_bad;    // smallest offending token index (diagnostic)
  int64_t count;        // counted (unmasked) tokens
  int64_t pad1;
  double loss_sum;
  double z_sum;
  double pad2[10];
};
static_assert(sizeof(Control) <= 256, "control block must fit its slot");
constexpr size_t kControlBytes = 256;

// Tile geometry the host planner needs (kept equal to the device traits).
constexpr int64_t kBf16TileM = 256;   // vocabulary rows per GEMM tile (bf16)
constexpr int64_t kComputeUnits = 256; // compute units of an MI355X (gfx950): one tile each per round
constexpr int64_t kBf16WaveM = 128;   // rows per forward partial (bf16)
constexpr int64_t kF64TileM = 128;
constexpr int64_t kF64PerCu = 2;      // fp64 workgroups resident per CU
constexpr int64_t kF64WaveM = 64;

// How one lce_forward / lce_backward call is laid out for a shape.
struct CEPlan {
  int32_t dtype = 0;          // LCE_BF16, LCE_F16 or LCE_F64
  int64_t n = 0, D = 0, V = 0, chunk = 0;
  size_t elem = 0;            // bytes per input element
  size_t acc = 0;             // bytes per accumulator element
  // forward
  int64_t wave_m = 0;         // vocabulary rows reduced into one partial
  int64_t n_vparts = 0;       // partials per token
  int64_t tok_per_pass = 0;   // tokens per forward launch
  // backward
  int64_t slab = 0;           // vocabulary rows per logit-gradient slab
  int64_t n_slabs = 0;
  int64_t d_ld = 0;           // row stride (tokens) of the slab buffer
  int64_t dh_splits = 0;      // split-K factor of the d_hidden product
  // bf16 slab pipeline (two slab buffers; one launch runs d_hidden and
  // d_weight of slab k with the logit gradient of slab k+1)
  int64_t pslab = 0;          // vocabulary rows per buffer
  int64_t pn_slabs = 0;
  int64_t pslab0 = 0;         // rows of the first slab (<= pslab; the others pslab)
  int64_t pdh_splits = 0;
  bool ppacked = false;       // launches packed onto the compute units (pack_tiles)
  // modelled duration (k-rows of a 256x256 tile on one compute unit) of the
  // two-call algorithm and of the single call that keeps the logits (16-bit
  // inputs; 0 when not modelled)
  int64_t model_two = 0, model_single = 0;
  double model_bwd_us = 0.0;  // packed-launch model of the 16-bit backward (us)
  // workspace layout (byte offsets)
  size_t off_partials = 0, off_zy = 0, off_losstok = 0;
  size_t off_dbuf = 0, off_dhacc = 0;
  size_t off_ht = 0;          // H^T [D][d_ld] (zero past n), the d_weight product's K-major operand
  size_t off_zyb = 0;         // bf16: target logits for the backward; 0 bytes for fp64
  size_t off_yloc = 0;        // [n] int64 shard-local target ids (shard calls)
  size_t total = 0;
  // Single-call forward+backward (16-bit inputs, every token in one chunk):
  // the logits of the whole batch are kept, [V][f_ld] fp32, and turned in
  // place into the bf16/fp16 logit gradient with row stride 2 * f_ld.
  bool f_ok = false;
  int64_t f_ld = 0;           // fp32 logit row stride (tokens)
  int64_t f_sp = 0;           // d_hidden split count (the reduction runs over all V)
  size_t off_fz = 0, off_fdh = 0, off_fht = 0, off_fyloc = 0;
  size_t f_total = 0;         // workspace of the single call (>= total)
};

// Tile counts per workgroup slot of a packed multi-product launch: slot
// b = 8 s + x is slot s of XCD x (the hardware deals workgroup b to XCD
// b % 8); it runs c[b][j] tiles of product j.
constexpr int kPackSlots = 256;
constexpr int kPackXcds = 8;
struct PackCounts {
  uint8_t c[kPackSlots][3];
};

// Packs the tiles of three independent products -- n[j] tiles of modelled
// duration dur[j] each (any unit), dealt to the XCDs in contiguous ranges --
// onto the 32 slots of every XCD so that the longest slot is as short as a
// best-fit-decreasing packing under a bisected makespan target gets it.
// *slots = slots used on the busiest XCD.  Returns false (and the caller
// keeps hardware dispatch) when a slot would hold more than 255 tiles of one
// product.
bool pack_tiles(const int64_t n[3], const double dur[3], PackCounts *out, int *slots,
                double *makespan = nullptr);

// Modelled duration (microseconds) of one 256 x 256 tile of each backward
// product on the 16-bit pipelined core: 1.43 us per 64-deep k-step of a
// K-major product and 1.71 for the MN-major d_hidden product, plus the
// epilogue and the pipeline fill (measured per tile at 2048 x 1024 x 151936).
inline double tile_us_dhidden(int64_t k_per_split) { return 11.8 + 1.71 * double((k_per_split + 63) / 64); }
inline double tile_us_dweight(int64_t n_tok) { return 5.2 + 1.43 * double((n_tok + 63) / 64); }
inline double tile_us_dlogit(int64_t d_model) { return 11.8 + 1.43 * double((d_model + 63) / 64); }
constexpr double kLaunchUs = 5.0;

// Fills *p; returns LCE_OK or a refusal status.
int32_t plan_ce(int64_t n, int64_t D, int64_t V, int64_t chunk, int32_t dtype, CEPlan *p);

struct DistillPlan {
  int64_t n = 0, V = 0;
  size_t off_rows = 0;        // per-row {loss, lse} doubles
  size_t total = 0;
};
int32_t plan_distill(int64_t n, int64_t V, DistillPlan *p);

bool finite_scalar(double x);
size_t dtype_size(int32_t dtype);

// Clears the control block and enqueues the target-range guard and the
// counted-token count (defined with the CE kernels); `stream` is a
// hipStream_t.
void launch_target_guard(const int64_t *targets, const uint8_t *mask, int64_t n, int64_t V,
                         Control *ctl, void *stream, lce_timers *tm);

// Brackets one launch of kernel kind `kind` with the caller's events.
struct TimedLaunch {
  lce_timer_slot *slot;
  void *stream;
  int32_t idx;
  TimedLaunch(lce_timers *t, int kind, void *st);
  ~TimedLaunch();
};

}  // namespace lce
