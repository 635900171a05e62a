// heuristic.cpp -- a zero-search default for a key that has no tuned entry
// while tuning is off: an analytic estimate of every candidate's time on the
// problem at hand, smallest first.
//
// The pages describe the untuned path as running a default kernel (the
// TunableOp guide's "tuning off" mode) and, as an adjacent design, a
// heuristic pick that costs no benchmark launches.  The estimate here is a
// roofline per candidate family with the quantisation of blocks over the
// CUs, the k-split's reduction pass and the transpose composites' extra
// pass; its constants are this library's own measurements on MI355X (the
// sustained fractions of the matrix-core peak of each tile family at large
// shapes, the streaming rates of the GEMV modes).  It is only a ranking:
// every candidate computes the same result, and a pick that turns out not
// to launch falls back to the naive kernel like a tuned winner does.
#include <algorithm>
#include <cmath>

#include "context.h"
#include "gt_internal.h"
#include "kernels/launchers.h"

namespace gt {

namespace {

constexpr double kHbmRate = 5.5e12;     // bytes/s, a long streaming read (measured 5.8e12)
constexpr double kCuFillRate = 1.0e11;  // bytes/s into one CU from L2 (measured at most 1.36e11)
constexpr double kLaunchS = 2.5e-6;     // one kernel launch back to back
constexpr double kBlockFillS = 1.0e-6;  // a block's pipeline fill and epilogue

// The datasheet's dense matrix-core peaks: the family efficiencies below are
// fractions of these (a measured peak already carries the board's power
// limit, which the efficiencies include too).
double peak_ops(int dtype) { return dtype == DT_F32 ? 157.3e12 : dtype == DT_E4M3 ? 5.0e15 : 2.5e15; }

// Fraction of the peak a tile family sustains in its main loop; smaller
// blocks read more LDS per flop and lose some of it.  The family, layout,
// wave grid and transposes come from the candidate's registration.
double tile_efficiency(const Candidate& c) {
  double e;
  if (c.dtype == DT_F32)
    e = 0.45;
  else if (c.family == TF_DMA16 && !c.xpose && c.layout == 0 && c.wn > 0 && c.BN / c.wn == 64)
    e = 0.52;  // NN with 8-byte reads of B
  else if (c.family == TF_DMA16)
    e = c.waves >= 8 ? 0.50 : 0.42;
  else if (c.family == TF_DMAH)
    e = 0.52;
  else if (c.family == TF_DMA && (c.xpose || c.layout == 1))
    e = 0.42;
  else if (c.family == TF_DMA)
    e = 0.34;  // an MN-major operand read with the slower transposing LDS reads
  else
    e = 0.30;  // register-staged tiles
  const int area = c.BM * c.BN;
  if (area < 256 * 256) e *= area >= 128 * 256 ? 0.9 : area >= 128 * 128 ? 0.75 : 0.55;
  return e;
}

double estimate_tile(const Candidate& c, const Problem& p, const DeviceState& d) {
  const double E = elem_bytes(p.in_dtype), Eo = elem_bytes(p.out_dtype);
  const int S = c.splitk > 1 ? tile_effective_splits(p.K, c.BK, c.splitk) : 1;
  const double kper = std::ceil((double)p.K / S);
  const double blocks = std::ceil((double)p.M / c.BM) * std::ceil((double)p.N / c.BN) * S;
  const double cus = d.cus > 0 ? d.cus : 256;
  const double rounds = std::ceil(blocks / cus);  // blocks one CU works through
  const double t_mma = rounds * 2.0 * c.BM * c.BN * kper / (peak_ops(p.in_dtype) / cus * tile_efficiency(c));
  double t_fill = rounds * (c.BM + c.BN) * kper * E / kCuFillRate;
  if (c.va_bytes > 0 && c.va_bytes < 16) t_fill *= 1.3;  // element-wise loads
  const double out_bytes = S > 1 ? 4.0 * S * p.M * p.N : Eo * p.M * p.N;
  const double t_hbm = ((double)(p.M + p.N) * p.K * E + out_bytes) / kHbmRate;
  double t = std::max(std::max(t_mma, t_fill), t_hbm) + rounds * kBlockFillS + kLaunchS;
  if (S > 1) t += 4.0 * S * p.M * p.N / kHbmRate + kLaunchS;  // the reduction pass
  if (c.xpose) {                                              // the transposes, read + write
    double bytes = 0;
    if (c.xpose & 1) bytes += 2.0 * p.M * p.K * E;
    if (c.xpose & 2) bytes += 2.0 * p.N * p.K * E;
    t += bytes / kHbmRate + kLaunchS;
  }
  return t;
}

double estimate_gemv(const Candidate& c, const Problem& p) {
  const double E = elem_bytes(p.in_dtype), Eo = elem_bytes(p.out_dtype);
  const double bytes = (double)p.K * p.N * E + (double)p.M * p.K * E + (double)p.M * p.N * Eo;
  // fraction of the 8 TB/s each reduction scheme streams B at
  double eff, extra = 0;
  switch (c.gemv_mode) {
    case 7: case 8: case 10: eff = 0.80; break;         // rhs stored N x K: one launch, no slices
    case 6: eff = 0.80; extra = kLaunchS; break;        // matrix cores, separate slice sum
    case 9: eff = 0.80; extra = kLaunchS + 1.0e-6; break;  // matrix cores, last slice sums: the
                                                            // per-workgroup L2 write-backs cost
                                                            // more than a second launch
    case 2: case 5: eff = 0.70; extra = kLaunchS; break;  // separate slice sum
    case 1: case 4: eff = 0.62; extra = 3.0e-6; break;    // last slice sums in the kernel
    default: eff = 0.45; break;                            // one workgroup walks all of K
  }
  return bytes / (8.0e12 * eff) + extra + kLaunchS;
}

}  // namespace

bool cand_aligned(const Candidate& c, const Problem& p) {
  const int E = elem_bytes(p.in_dtype);
  if (c.va_bytes > 1 && ((reinterpret_cast<uintptr_t>(p.A) % c.va_bytes) != 0 || (p.lda * E) % c.va_bytes != 0))
    return false;
  if (c.vb_bytes > 1 && ((reinterpret_cast<uintptr_t>(p.B) % c.vb_bytes) != 0 || (p.ldb * E) % c.vb_bytes != 0))
    return false;
  return true;
}

double default_estimate_s(const Candidate& c, const Problem& p, const DeviceState& d) {
  if (c.group == G_NAIVE) return 2.0 * p.M * p.N * p.K / 2.0e12;  // one thread per output
  if (c.group == G_GEMV) return estimate_gemv(c, p);
  return estimate_tile(c, p, d);
}

int default_candidate(int dtype, const KeyFields& k, const Problem& p, const DeviceState& d) {
  const std::vector<Candidate>& set = candidates(dtype);
  int best = 0;
  double best_t = INFINITY;
  for (size_t i = 1; i < set.size(); ++i) {
    const Candidate& c = set[i];
    if (cand_priority(c, k) == P_NEVER || !cand_supported(c, k) || !cand_aligned(c, p)) continue;
    double t = default_estimate_s(c, p, d);
    if (cand_priority(c, k) < P_HIGH) t *= 1.05;  // the plan's own lower tier (narrow loads, ill-fitting GEMV rows)
    if (t < best_t) {
      best_t = t;
      best = (int)i;
    }
  }
  return best;
}

}  // namespace gt
