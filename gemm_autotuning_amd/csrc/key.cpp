// key.cpp -- the tuning key (Burn "autotune" page, section on the tuning key:
// shape bucketing).
//
// m, n, k are rounded up to their bucket: the smallest power of the level's
// base not below the dimension, rounded up to an integer (base 2 at the
// balanced level, 2.5 at the minimal level, 1.5 at the extensive level),
// unchanged at the full level.  The pow2 factors are the trailing zero
// bits of the bucketed k (lhs) and n (rhs), at most 4.  The stride factors are
// the trailing zero bits of the real leading dimension in bytes, at most 10
// (a leading dimension of 0 counts as 10): they decide which vector-load
// widths a kernel may use.  Element types and the two layouts are part of the
// key, as are the size class (Small if every bucketed dim is below 512, Medium
// below 2048, else Large) and the shape class of the real dims.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "gt_internal.h"

namespace gt {

// The power is formed as a product of factors of the base in double
// precision, one rounding per factor, then rounded up to an integer; buckets
// beyond the 32-bit range are clamped to its top.
static uint32_t anchor(int64_t x, int level) {
  const double top = 4294967295.0;
  if (level == LEVEL_FULL) return x > (int64_t)0xffffffffLL ? 0xffffffffu : (uint32_t)x;
  const double base = level == LEVEL_MINIMAL ? 2.5 : level == LEVEL_EXTENSIVE ? 1.5 : 2.0;
  double v = 1.0;
  while (v < (double)x) v *= base;
  v = ceil(v);
  return v > top ? 0xffffffffu : (uint32_t)v;
}

const char* level_name(int level) {
  switch (level) {
    case LEVEL_FULL: return "full";
    case LEVEL_MINIMAL: return "minimal";
    case LEVEL_EXTENSIVE: return "extensive";
    default: return "balanced";
  }
}

int level_from_name(const char* name) {
  for (int l : {LEVEL_BALANCED, LEVEL_FULL, LEVEL_MINIMAL, LEVEL_EXTENSIVE})
    if (!strcmp(name, level_name(l))) return l;
  return -1;
}

const int kWildcardOrder[7] = {1, 2, 4, 3, 5, 6, 7};

KeyFields mask_key(const KeyFields& f, int mask) {
  KeyFields g = f;
  if (mask & 1) g.m = 0;
  if (mask & 2) g.n = 0;
  if (mask & 4) g.k = 0;
  return g;
}

static int ctz64(uint64_t x) { return x ? __builtin_ctzll(x) : 64; }

static uint8_t stride_factor(int64_t ld, int eb) {
  if (ld == 0) return 10;
  int t = ctz64((uint64_t)ld * (uint64_t)eb);
  return (uint8_t)(t > 10 ? 10 : t);
}

static uint8_t kind_of(int64_t M, int64_t N, int64_t K) {
  if (K == 1) {
    if (M == 1) return KIND_SCALARVEC;
    if (N == 1) return KIND_VECSCALAR;
    return KIND_OUTER;
  }
  if (M == 1 && N == 1) return KIND_INNER;
  if (M == 1) return KIND_VECMAT;
  if (N == 1) return KIND_MATVEC;
  return KIND_GENERAL;
}

KeyFields make_key_fields(const Problem& p, int level) {
  KeyFields f;
  memset(&f, 0, sizeof(f));
  f.m = anchor(p.M, level);
  f.n = anchor(p.N, level);
  f.k = anchor(p.K, level);
  int tk = ctz64(f.k), tn = ctz64(f.n);
  f.lhs_pow2 = (uint8_t)(tk > 4 ? 4 : tk);
  f.rhs_pow2 = (uint8_t)(tn > 4 ? 4 : tn);
  const int eb = elem_bytes(p.in_dtype);
  f.lhs_stride = stride_factor(p.lda, eb);
  f.rhs_stride = stride_factor(p.ldb, eb);
  f.elem_lhs = f.elem_rhs = (uint8_t)p.in_dtype;
  f.elem_out = (uint8_t)p.out_dtype;
  f.layout_lhs = p.ta ? 1 : 0;
  f.layout_rhs = p.tb ? 1 : 0;
  if (f.m < 512 && f.n < 512 && f.k < 512)
    f.scale = SCALE_SMALL;
  else if (f.m < 2048 && f.n < 2048 && f.k < 2048)
    f.scale = SCALE_MEDIUM;
  else
    f.scale = SCALE_LARGE;
  f.kind = kind_of(p.M, p.N, p.K);
  return f;
}

Key pack_key(const KeyFields& f) {
  uint8_t b[32];
  memset(b, 0, sizeof(b));
  const uint32_t d[3] = {f.m, f.n, f.k};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 4; ++j) b[4 * i + j] = (uint8_t)(d[i] >> (8 * j));
  const uint8_t t[11] = {f.lhs_pow2, f.lhs_stride, f.rhs_pow2,  f.rhs_stride, f.elem_lhs, f.elem_rhs,
                         f.elem_out, f.layout_lhs, f.layout_rhs, f.scale,      f.kind};
  memcpy(b + 12, t, 11);
  Key k;
  memcpy(k.w, b, 32);
  return k;
}

KeyFields unpack_key(const Key& k) {
  uint8_t b[32];
  memcpy(b, k.w, 32);
  KeyFields f;
  uint32_t d[3];
  for (int i = 0; i < 3; ++i) d[i] = b[4 * i] | (b[4 * i + 1] << 8) | (b[4 * i + 2] << 16) | ((uint32_t)b[4 * i + 3] << 24);
  f.m = d[0];
  f.n = d[1];
  f.k = d[2];
  f.lhs_pow2 = b[12];
  f.lhs_stride = b[13];
  f.rhs_pow2 = b[14];
  f.rhs_stride = b[15];
  f.elem_lhs = b[16];
  f.elem_rhs = b[17];
  f.elem_out = b[18];
  f.layout_lhs = b[19];
  f.layout_rhs = b[20];
  f.scale = b[21];
  f.kind = b[22];
  return f;
}

static const char* kDtypeNames[4] = {"f32", "f16", "bf16", "e4m3"};
static const char* kScaleNames[3] = {"Small", "Medium", "Large"};
static const char* kKindNames[7] = {"General", "MatVec", "VecMat", "ScalarVec", "VecScalar", "InnerProduct", "OuterProduct"};
static const char* kLayoutCompact[2] = {"Contiguous", "MildlyPermuted{transposed:true;batch_swap:false}"};
static const char* kLayoutDisplay[2] = {"Contiguous", "MildlyPermuted { transposed: true, batch_swap: false }"};

static std::string dim_text(uint32_t v) { return v ? std::to_string(v) : std::string("*"); }

static std::string render(const KeyFields& f, const char* const* layouts) {
  char buf[512];
  snprintf(buf, sizeof(buf),
           "m=%s n=%s k=%s lhs_pow2=%u lhs_stride=%u rhs_pow2=%u rhs_stride=%u elem_lhs=%s elem_rhs=%s elem_out=%s "
           "layout_lhs=%s layout_rhs=%s scale=%s kind=%s",
           dim_text(f.m).c_str(), dim_text(f.n).c_str(), dim_text(f.k).c_str(), f.lhs_pow2, f.lhs_stride, f.rhs_pow2, f.rhs_stride, kDtypeNames[f.elem_lhs & 3],
           kDtypeNames[f.elem_rhs & 3], kDtypeNames[f.elem_out & 3], layouts[f.layout_lhs & 1],
           layouts[f.layout_rhs & 1], kScaleNames[f.scale % 3], kKindNames[f.kind % 7]);
  return buf;
}

std::string key_compact(const KeyFields& f) { return render(f, kLayoutCompact); }
std::string key_display(const KeyFields& f) { return render(f, kLayoutDisplay); }

static bool parse_uint(const std::string& s, uint32_t* out) {
  if (s.empty() || s.size() > 10) return false;
  uint64_t v = 0;
  for (char c : s) {
    if (c < '0' || c > '9') return false;
    v = v * 10 + (uint64_t)(c - '0');
  }
  if (v > 0xffffffffull) return false;
  *out = (uint32_t)v;
  return true;
}

static int lookup(const std::string& v, const char* const* names, int n) {
  for (int i = 0; i < n; ++i)
    if (v == names[i]) return i;
  return -1;
}

bool key_parse_compact(const std::string& s, KeyFields* out) {
  static const char* kFields[14] = {"m",        "n",        "k",          "lhs_pow2",   "lhs_stride",
                                    "rhs_pow2", "rhs_stride", "elem_lhs", "elem_rhs",   "elem_out",
                                    "layout_lhs", "layout_rhs", "scale",  "kind"};
  std::vector<std::string> toks;
  size_t pos = 0;
  while (pos <= s.size()) {
    size_t sp = s.find(' ', pos);
    if (sp == std::string::npos) sp = s.size();
    toks.push_back(s.substr(pos, sp - pos));
    pos = sp + 1;
  }
  if (toks.size() != 14) return false;
  KeyFields f;
  memset(&f, 0, sizeof(f));
  uint32_t num[7];
  for (int i = 0; i < 14; ++i) {
    const std::string& t = toks[i];
    size_t eq = t.find('=');
    if (eq == std::string::npos || t.substr(0, eq) != kFields[i]) return false;
    std::string v = t.substr(eq + 1);
    if (i < 3 && v == "*") {
      num[i] = 0;  // wildcard
    } else if (i < 7) {
      if (!parse_uint(v, &num[i])) return false;
      if (i < 3 && num[i] == 0) return false;
      if (i >= 3 && num[i] > 255) return false;
    } else if (i < 10) {
      int d = lookup(v, kDtypeNames, 4);
      if (d < 0) return false;
      (i == 7 ? f.elem_lhs : i == 8 ? f.elem_rhs : f.elem_out) = (uint8_t)d;
    } else if (i < 12) {
      int l = lookup(v, kLayoutCompact, 2);
      if (l < 0) return false;
      (i == 10 ? f.layout_lhs : f.layout_rhs) = (uint8_t)l;
    } else if (i == 12) {
      int sc = lookup(v, kScaleNames, 3);
      if (sc < 0) return false;
      f.scale = (uint8_t)sc;
    } else {
      int kd = lookup(v, kKindNames, 7);
      if (kd < 0) return false;
      f.kind = (uint8_t)kd;
    }
  }
  f.m = num[0];
  f.n = num[1];
  f.k = num[2];
  f.lhs_pow2 = (uint8_t)num[3];
  f.lhs_stride = (uint8_t)num[4];
  f.rhs_pow2 = (uint8_t)num[5];
  f.rhs_stride = (uint8_t)num[6];
  *out = f;
  return true;
}

}  // namespace gt
