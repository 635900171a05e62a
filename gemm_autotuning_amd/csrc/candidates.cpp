// candidates.cpp -- the candidate set of each input type and the key-only
// rules that order it.
//
// Registration order is the index order (and the order the checksum hashes):
// the naive kernel first (the fallback that always works, as the Burn
// "autotune" page's first candidate is), then the GEMV kernels, then the tile
// kernels of tile_registry.inc (split-K ones expanded over their slice
// counts).
//
// The page's table of group rules did not survive extraction, so the rules
// below are this library's own reading, chosen so the knowledge that M = 1
// wants a streaming GEMV, that huge tiles waste work on small problems, and
// that a small output with a long K wants a k-split, is encoded in priorities
// the way the page describes (priority per group and per candidate, functions
// of the key; negative = skip for this key; unsupported = demoted to MIN).
#include <stdio.h>
#include <string.h>

#include "gt_internal.h"

#include "gemv_decls.inc"
#include "tile_decls.inc"

namespace gt {

namespace {

struct TileEntry {
  const char* name;
  int dtype, layout, BM, BN, BK, WM, WN, ST, va_bytes, vb_bytes, splitk, lds;
  int xpose;  // operands transposed into the workspace first: 1 lhs, 2 rhs
  int family;  // TileFamily
  int wk;      // k-groups of WM x WN waves per block
  LaunchFn fn;
};

const TileEntry kTiles[] = {
#include "tile_registry.inc"
};

// name, input type, rows, column block, waves, rhs load bytes, mode (0 whole
// K per workgroup, 1 last-slice reduction, 2 separate reduction pass, 3 XCD
// stream, 4 flat with last-slice reduction, 5 flat with a separate reduction
// pass), slices, rows per load step, LDS bytes, launcher
struct GemvEntry {
  const char* name;
  int dtype, rows, cw, nw, vb_bytes, mode, splits, rows_per_step, lds;
  LaunchFn fn;
};

const GemvEntry kGemv[] = {
#include "gemv_registry.inc"
};

const int kSplitCounts[] = {4, 8, 16, 32, 64};

std::vector<Candidate> build_set(int dtype) {
  std::vector<Candidate> out;
  Candidate nv;
  nv.name = "naive";
  nv.dtype = dtype;
  nv.group = G_NAIVE;
  nv.in_tile_group = false;
  nv.layout = -1;
  nv.BM = nv.BN = 16;
  nv.BK = 1;
  nv.waves = 4;
  nv.wm = nv.wn = 0;
  nv.stages = 0;
  nv.splitk = 1;
  nv.va_bytes = nv.vb_bytes = 0;
  nv.rows = 0;
  nv.cw = nv.rows_per_step = nv.gemv_mode = 0;
  nv.lds_bytes = 0;
  nv.xpose = 0;
  nv.family = TF_NONE;
  nv.launch = &launch_naive;
  out.push_back(nv);
  for (const GemvEntry& g : kGemv) {
    if (g.dtype != dtype) continue;
    Candidate c;
    c.name = g.name;
    c.dtype = dtype;
    c.group = G_GEMV;
    c.in_tile_group = true;
    c.layout = (g.mode == 7 || g.mode == 8 || g.mode == 10) ? -3 : -2;  // rhs stored transposed (7, 8, 10) or as is
    c.BM = g.rows;
    c.BN = g.cw;
    c.BK = 0;
    c.waves = g.nw;
    c.wm = c.wn = 0;
    c.stages = 0;
    c.splitk = g.splits;
    c.va_bytes = 0;
    c.vb_bytes = g.vb_bytes;
    c.rows = g.rows;
    c.cw = g.cw;
    c.rows_per_step = g.rows_per_step;
    c.gemv_mode = g.mode;
    c.lds_bytes = g.lds;
    c.xpose = 0;
    c.family = TF_NONE;
    c.launch = g.fn;
    out.push_back(c);
  }
  for (const TileEntry& t : kTiles) {
    if (t.dtype != dtype) continue;
    Candidate c;
    c.dtype = dtype;
    c.group = G_TILE;
    c.in_tile_group = true;
    c.layout = t.layout;
    c.BM = t.BM;
    c.BN = t.BN;
    c.BK = t.BK;
    c.waves = t.WM * t.WN * t.wk;
    c.wm = t.WM;
    c.wn = t.WN;
    c.stages = t.ST;
    c.va_bytes = t.va_bytes;
    c.vb_bytes = t.vb_bytes;
    c.rows = 0;
    c.cw = c.rows_per_step = c.gemv_mode = 0;
    c.lds_bytes = t.lds;
    c.xpose = t.xpose;
    c.family = t.family;
    c.launch = t.fn;
    if (!t.splitk) {
      c.name = t.name;
      c.splitk = 1;
      out.push_back(c);
    } else {
      for (int s : kSplitCounts) {
        char buf[160];
        snprintf(buf, sizeof(buf), "%s_k%d", t.name, s);
        c.name = buf;
        c.splitk = s;
        out.push_back(c);
      }
    }
  }
  return out;
}

struct Sets {
  std::vector<Candidate> v[4];
  std::string sum[4];
  Sets() {
    for (int d = 0; d < 4; ++d) {
      v[d] = build_set(d);
      // 64-bit FNV-1a over the names joined by '\n'
      uint64_t h = 0xCBF29CE484222325ull;
      for (size_t i = 0; i < v[d].size(); ++i) {
        if (i) {
          h ^= (uint8_t)'\n';
          h *= 0x100000001B3ull;
        }
        for (unsigned char ch : v[d][i].name) {
          h ^= ch;
          h *= 0x100000001B3ull;
        }
      }
      char buf[17];
      snprintf(buf, sizeof(buf), "%016llx", (unsigned long long)h);
      sum[d] = buf;
    }
  }
};

const Sets& sets() {
  static const Sets s;
  return s;
}

bool layout_ok(const Candidate& c, int layout) {
  if (c.layout == -1) return true;
  if (c.layout == -2) return (layout & 1) == 0;  // rhs not transposed
  if (c.layout == -3) return (layout & 1) != 0;  // rhs transposed
  return c.layout == layout;
}

int log2i(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

// The wide sibling of a narrow-load candidate can run when both stride
// factors allow 16-byte rows.
bool wide_allowed(const KeyFields& k) { return k.lhs_stride >= 4 && k.rhs_stride >= 4; }

bool is_narrow(const Candidate& c) {
  if (c.group == G_NAIVE) return false;
  if (c.group == G_GEMV) return c.vb_bytes < 16 && c.dtype != DT_F32;
  return c.va_bytes < 16 || c.vb_bytes < 16;
}

}  // namespace

const std::vector<Candidate>& candidates(int dtype) {
  static const std::vector<Candidate> empty;
  if (dtype < 0 || dtype > 3) return empty;
  return sets().v[dtype];
}

std::string candidate_checksum(int dtype) { return (dtype < 0 || dtype > 3) ? std::string() : sets().sum[dtype]; }

int find_candidate(int dtype, const std::string& name) {
  const std::vector<Candidate>& s = candidates(dtype);
  for (size_t i = 0; i < s.size(); ++i)
    if (s[i].name == name) return (int)i;
  return -1;
}

int group_priority(int group, const KeyFields& k) {
  switch (group) {
    case G_NAIVE: return P_MIN;
    case G_GEMV: return k.m == 1 ? P_MAX : P_NEVER;
    case G_TILE: return P_HIGH;
  }
  return P_NEVER;
}

int cand_priority(const Candidate& c, const KeyFields& k) {
  const int layout = (k.layout_lhs ? 2 : 0) | (k.layout_rhs ? 1 : 0);
  if (!layout_ok(c, layout)) return P_NEVER;
  if (c.group == G_NAIVE) return P_MIN;
  const int narrow_prio = (is_narrow(c) && wide_allowed(k)) ? P_MEDIUM : P_HIGH;
  if (c.group == G_GEMV) {
    if ((uint32_t)c.rows < k.m) return P_NEVER;
    // the smallest row count of this type's GEMV kernels for this layout
    // that covers m is the natural fit; larger ones only waste lanes
    uint32_t fit = 0xffffffffu;
    for (const Candidate& o : candidates(c.dtype))
      if (o.group == G_GEMV && layout_ok(o, layout) && (uint32_t)o.rows >= k.m && (uint32_t)o.rows < fit)
        fit = (uint32_t)o.rows;
    const int p = (uint32_t)c.rows == fit ? P_HIGH : P_MEDIUM;
    return p < narrow_prio ? p : narrow_prio;
  }
  // tiles
  if (c.splitk > 1) {
    const uint64_t tiles = (uint64_t)((k.m + c.BM - 1) / c.BM) * (uint64_t)((k.n + c.BN - 1) / c.BN);
    if (tiles > 64 || (uint64_t)k.k < (uint64_t)4 * c.splitk * c.BK) return P_NEVER;
    return narrow_prio;
  }
  if (c.BM * c.BN <= 32 * 32) {  // k-group blocks: few blocks, a short walk of k-tiles
    const uint64_t tiles = (uint64_t)((k.m + c.BM - 1) / c.BM) * (uint64_t)((k.n + c.BN - 1) / c.BN);
    if (tiles > 256 || (uint64_t)k.k > (uint64_t)4 * c.BK) return P_NEVER;
  }
  int p = P_HIGH;
  if ((c.BM > 64 && (uint32_t)c.BM >= 2 * k.m) || (c.BN > 64 && (uint32_t)c.BN >= 2 * k.n)) p = P_MEDIUM;
  return p < narrow_prio ? p : narrow_prio;
}

bool cand_supported(const Candidate& c, const KeyFields& k) {
  if (c.va_bytes > 1 && k.lhs_stride < log2i(c.va_bytes)) return false;
  if (c.vb_bytes > 1 && k.rhs_stride < log2i(c.vb_bytes)) return false;
  if (c.lds_bytes > 160 * 1024) return false;
  if ((int)k.elem_out == DT_E4M3) return false;
  return true;
}

size_t cand_workspace(const Candidate& c, const Problem& p) {
  if (c.group == G_GEMV) {
    if (c.gemv_mode == 0 || c.gemv_mode == 7 || c.gemv_mode == 8 || c.gemv_mode == 10) return 0;  // no partials
    if (c.gemv_mode >= 4) {          // one K slice per rows_per_step rows
      const int64_t s4 = (p.K + c.rows_per_step - 1) / c.rows_per_step;
      return s4 > 1 ? gemv_workspace_bytes(p.M, p.N, (int)s4, (int)((p.N + c.cw - 1) / c.cw)) : 0;
    }
    const int s = gemv_effective_splits(p.K, c.splitk, c.rows_per_step);
    return gemv_workspace_bytes(p.M, p.N, s, (int)((p.N + c.cw - 1) / c.cw));
  }
  if (c.group == G_TILE && c.splitk > 1) return tile_splitk_workspace_bytes(p.M, p.N, p.K, c.BK, c.splitk);
  if (c.xpose) return tile_xpose_workspace_bytes(p.M, p.N, p.K, elem_bytes(c.dtype), c.xpose & 1, c.xpose & 2);
  return 0;
}

PlanInput plan_input_for(int dtype, const KeyFields& k) {
  PlanInput in;
  for (int g = 0; g < N_GROUPS; ++g) in.group_prio.push_back(group_priority(g, k));
  for (const Candidate& c : candidates(dtype)) {
    std::vector<int> gs;
    gs.push_back(c.group);
    if (c.group == G_GEMV && c.in_tile_group) gs.push_back(G_TILE);
    in.cand_groups.push_back(gs);
    in.cand_prio.push_back(cand_priority(c, k));
    in.supported.push_back(cand_supported(c, k));
  }
  return in;
}

}  // namespace gt
