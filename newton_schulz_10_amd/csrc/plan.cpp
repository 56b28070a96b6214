// Host-side planning and argument validation (see plan.h).
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <sstream>
#include <tuple>

namespace muon {

namespace {
size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
}  // namespace

int pad_granularity_m(muon_dtype dtype) { return dtype == MUON_BF16 ? 128 : 64; }
int pad_granularity_n(muon_dtype dtype) { return dtype == MUON_BF16 ? 256 : 64; }

size_t dtype_size(muon_dtype dtype) { return dtype == MUON_BF16 ? 2 : 4; }

Layout batch_layout(int count, int m_pad, int n_pad, muon_dtype dtype) {
  Layout L;
  const size_t es = dtype_size(dtype);
  const size_t A = 512;
  L.mat_x = (size_t)m_pad * (size_t)n_pad;
  L.mat_a = (size_t)m_pad * (size_t)m_pad;
  L.ew_blocks = (m_pad / kEwTile) * (n_pad / kEwTile);
  size_t off = 0;
  L.x0 = off;       off = align_up(off + (size_t)count * L.mat_x * es, A);
  L.x1 = off;       off = align_up(off + (size_t)count * L.mat_x * es, A);
  L.a = off;        off = align_up(off + (size_t)count * L.mat_a * es, A);
  L.b = off;        off = align_up(off + (size_t)count * L.mat_a * es, A);
  L.partials = off; off = align_up(off + (size_t)count * (size_t)L.ew_blocks * sizeof(float), A);
  L.nonzero = off;  off = align_up(off + (size_t)count * (size_t)L.ew_blocks * sizeof(int), A);
  L.scales = off;   off = align_up(off + (size_t)count * sizeof(float), A);
  L.live = off;     off = align_up(off + (size_t)count * sizeof(int), A);
  L.live_list = off; off = align_up(off + (size_t)count * sizeof(int), A);
  L.nlive = off;    off = align_up(off + sizeof(int), A);
  L.ptab = off;     off = align_up(off + (size_t)count * 16, A);   // fused-apply entries
  L.sched = off;    off = align_up(off + (size_t)kSchedWords * sizeof(int), A);
  L.total = off;
  return L;
}

int check_shape(int m, int n, std::string& err, int index) {
  if (m < 1 || n < 1 || m > MUON_MAX_DIM || n > MUON_MAX_DIM) {
    std::ostringstream s;
    s << "matrix";
    if (index >= 0) s << " " << index;
    s << ": shape " << m << " x " << n << " outside [1, " << MUON_MAX_DIM << "]";
    err = s.str();
    return MUON_ERR_INVALID_ARGUMENT;
  }
  return MUON_OK;
}

// Estimated time of the three NS GEMMs of one bf16 batch of c matrices on
// `cus` compute units, in units of one K element of one tile. It follows the
// bf16 GEMM's geometry: 256 x 256 tiles plus, when m_pad = 256 F + 128, wide
// 128 x 512 tiles for the half row; Gram and Poly over the lower triangle.
// Tiles are split into 8 equal per-XCD ranges, each worked in rounds by
// cus/8 workgroups; a tile costs its K plus an epilogue/prologue allowance,
// a launch a quarter of that.
static double ns_batch_cost(long long c, int m_pad, int n_pad, int cus) {
  const long long F = m_pad / 256, half = (m_pad % 256) != 0;
  const long long slots = (long long)(cus / 8) * 8;
  auto rounds = [&](long long tiles) -> long long {
    if (slots < 8 || tiles <= slots) return 1;
    const long long per_xcd = (tiles + 7) / 8;
    return (per_xcd + slots / 8 - 1) / (slots / 8);
  };
  const long long ts = F + half, tu = n_pad / 256;
  const long long sym = (F * (F + 1) / 2 + (half ? (ts + 1) / 2 : 0)) * c;
  const long long upd = (F * tu + (half ? (tu + 1) / 2 : 0)) * c;
  const double E = 640.0;   // epilogue + prologue of a tile, in K elements
  const double L = 256.0;   // one launch
  return rounds(sym) * (n_pad + E) + rounds(sym) * (m_pad + E) + rounds(upd) * (m_pad + E) + 3 * L;
}

int build_plan(const int* rows, const int* cols, int num, muon_dtype dtype, size_t cap, int cus,
               Plan& out, std::string& err, const int* set_of, int num_sets, size_t max_ws) {
  out = Plan();
  if (num < 0) { err = "num < 0"; return MUON_ERR_INVALID_ARGUMENT; }
  if (num > 0 && (!rows || !cols)) { err = "rows/cols array is NULL"; return MUON_ERR_INVALID_ARGUMENT; }
  if (dtype != MUON_F32 && dtype != MUON_BF16) { err = "unknown dtype"; return MUON_ERR_INVALID_ARGUMENT; }
  if (cap == 0) cap = MUON_DEFAULT_BATCH_CAP;
  if (set_of && num_sets < 1) { err = "coefficient sets given with num_sets < 1"; return MUON_ERR_INVALID_ARGUMENT; }
  out.transposed.resize(num);
  // key = (min, max, set); groups keep first-appearance order of their
  // matrices.
  std::map<std::tuple<int, int, int>, std::vector<int>> groups;
  for (int i = 0; i < num; ++i) {
    int rc = check_shape(rows[i], cols[i], err, i);
    if (rc) return rc;
    const int set = set_of ? set_of[i] : 0;
    if (set < 0 || (set_of && set >= num_sets)) {
      std::ostringstream s;
      s << "matrix " << i << ": coefficient set " << set << " outside [0, " << num_sets << ")";
      err = s.str();
      return MUON_ERR_INVALID_ARGUMENT;
    }
    out.transposed[i] = rows[i] > cols[i] ? 1 : 0;
    groups[{std::min(rows[i], cols[i]), std::max(rows[i], cols[i]), set}].push_back(i);
  }
  // Descending element count (large matrices first); ties: larger long
  // side first, then larger short side, then lower set index.
  std::vector<std::pair<std::tuple<int, int, int>, std::vector<int>>> g(groups.begin(), groups.end());
  std::stable_sort(g.begin(), g.end(), [](const auto& x, const auto& y) {
    const int xm = std::get<0>(x.first), xn = std::get<1>(x.first), ym = std::get<0>(y.first),
              yn = std::get<1>(y.first);
    long long ex = (long long)xm * xn;
    long long ey = (long long)ym * yn;
    if (ex != ey) return ex > ey;
    if (xn != yn) return xn > yn;
    if (xm != ym) return xm > ym;
    return std::get<2>(x.first) < std::get<2>(y.first);
  });
  const int pgm = pad_granularity_m(dtype), pgn = pad_granularity_n(dtype);
  size_t ws = 0;
  for (size_t gi = 0; gi < g.size(); ++gi) {
    const int m = std::get<0>(g[gi].first), n = std::get<1>(g[gi].first), set = std::get<2>(g[gi].first);
    const std::vector<int>& idx = g[gi].second;
    const int cnt = (int)idx.size();
    const size_t per_mat = (size_t)m * (size_t)n;
    size_t per_batch = std::max<size_t>(1, cap / per_mat);
    const int m_pad = (int)round_up(m, pgm), n_pad = (int)round_up(n, pgn);
    if (max_ws > 0) {
      // Workspace bound: the largest count whose batch layout fits.
      if (batch_layout(1, m_pad, n_pad, dtype).total > max_ws) {
        std::ostringstream s;
        s << "matrix " << idx[0] << " (" << rows[idx[0]] << " x " << cols[idx[0]] << ") needs "
          << batch_layout(1, m_pad, n_pad, dtype).total << " bytes of workspace, more than the "
          << max_ws << " available";
        err = s.str();
        return MUON_ERR_INVALID_ARGUMENT;
      }
      size_t lo = 1, hi = std::min<size_t>(per_batch, (size_t)cnt);
      while (lo < hi) {
        const size_t mid = (lo + hi + 1) / 2;
        if (batch_layout((int)mid, m_pad, n_pad, dtype).total <= max_ws) lo = mid; else hi = mid - 1;
      }
      per_batch = lo;
    }
    int nb = (int)((cnt + per_batch - 1) / per_batch);
    if (dtype == MUON_BF16 && cus > 0 && cnt > 1 && max_ws == 0) {
      // Up to four more batches than needed, if their tiles fill the
      // compute units' rounds better (balanced sizes, as below).
      double best = 0.0;
      int best_nb = nb;
      for (int t = nb; t <= std::min(cnt, nb + 4); ++t) {
        double cost = 0.0;
        for (int b = 0; b < t; ++b) cost += ns_batch_cost(cnt / t + (b < cnt % t ? 1 : 0), m_pad, n_pad, cus);
        if (t == nb || cost < best) { best = cost; best_nb = t; }
      }
      nb = best_nb;
    }
    int start = 0;
    for (int b = 0; b < nb; ++b) {
      int c = cnt / nb + (b < cnt % nb ? 1 : 0);  // balanced sizes
      Batch B{(int)gi, m, n, m_pad, n_pad, (int)out.order.size(), c, set};
      for (int k = 0; k < c; ++k) out.order.push_back(idx[start + k]);
      start += c;
      out.batches.push_back(B);
      ws = std::max(ws, batch_layout(c, m_pad, n_pad, dtype).total);
    }
  }
  out.workspace_bytes = ws;
  return MUON_OK;
}

void default_options(muon_options& o) {
  o.nesterov = 1;
  o.momentum_form = 0;
  o.weight_decay = 0.0f;
  o.scale_rule = 0;
  o.rms_target = 0.2f;
  o.eps = 1e-7f;
  o.coeffs = nullptr;
  o.batch_cap_elems = MUON_DEFAULT_BATCH_CAP;
  o.compute_units = 0;
  o.ns_dtype = -1;
  o.poly_form = MUON_POLY_SQUARE;
  o.num_coeff_sets = 0;
  o.coeff_sets = nullptr;
  o.coeff_set_of = nullptr;
}

int check_options(const muon_options& o, int ns_steps, std::string& err) {
  if (o.nesterov != 0 && o.nesterov != 1) { err = "options.nesterov must be 0 or 1"; return MUON_ERR_INVALID_ARGUMENT; }
  if (o.momentum_form != 0 && o.momentum_form != 1) { err = "options.momentum_form must be 0 or 1"; return MUON_ERR_INVALID_ARGUMENT; }
  if (o.scale_rule < 0 || o.scale_rule > 2) { err = "options.scale_rule must be 0, 1 or 2"; return MUON_ERR_INVALID_ARGUMENT; }
  if (!std::isfinite(o.weight_decay)) { err = "options.weight_decay is not finite"; return MUON_ERR_INVALID_ARGUMENT; }
  if (!std::isfinite(o.rms_target)) { err = "options.rms_target is not finite"; return MUON_ERR_INVALID_ARGUMENT; }
  if (!(o.eps >= 0.0f) || !std::isfinite(o.eps)) { err = "options.eps must be finite and >= 0"; return MUON_ERR_INVALID_ARGUMENT; }
  if (o.compute_units < -1) { err = "options.compute_units must be >= -1"; return MUON_ERR_INVALID_ARGUMENT; }
  if (o.ns_dtype != -1 && o.ns_dtype != MUON_F32 && o.ns_dtype != MUON_BF16) {
    err = "options.ns_dtype must be -1, MUON_F32 or MUON_BF16"; return MUON_ERR_INVALID_ARGUMENT;
  }
  if (o.coeffs) {
    for (int i = 0; i < 3 * ns_steps; ++i)
      if (!std::isfinite(o.coeffs[i])) {
        std::ostringstream s; s << "options.coeffs[" << i << "] is not finite"; err = s.str();
        return MUON_ERR_INVALID_ARGUMENT;
      }
  }
  if (o.poly_form != MUON_POLY_DIRECT && o.poly_form != MUON_POLY_SQUARE && o.poly_form != MUON_POLY_FOLDED) {
    err = "options.poly_form must be MUON_POLY_DIRECT, MUON_POLY_SQUARE or MUON_POLY_FOLDED";
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (o.num_coeff_sets < 0) { err = "options.num_coeff_sets must be >= 0"; return MUON_ERR_INVALID_ARGUMENT; }
  if (o.num_coeff_sets > 0) {
    if (o.coeffs) { err = "options.coeffs must be NULL when num_coeff_sets > 0"; return MUON_ERR_INVALID_ARGUMENT; }
    if (!o.coeff_sets || !o.coeff_set_of) {
      err = "options.coeff_sets and options.coeff_set_of are required when num_coeff_sets > 0";
      return MUON_ERR_INVALID_ARGUMENT;
    }
    const long long total = 3LL * ns_steps * o.num_coeff_sets;
    for (long long i = 0; i < total; ++i)
      if (!std::isfinite(o.coeff_sets[i])) {
        std::ostringstream s; s << "options.coeff_sets[" << i << "] is not finite"; err = s.str();
        return MUON_ERR_INVALID_ARGUMENT;
      }
  }
  return MUON_OK;
}

int check_scalars(float lr, float beta, int ns_steps, muon_dtype dtype, std::string& err) {
  if (!std::isfinite(lr)) { err = "lr is not finite"; return MUON_ERR_INVALID_ARGUMENT; }
  if (!std::isfinite(beta)) { err = "beta is not finite"; return MUON_ERR_INVALID_ARGUMENT; }
  if (ns_steps < 0 || ns_steps > MUON_MAX_NS_STEPS) {
    std::ostringstream s; s << "ns_steps " << ns_steps << " outside [0, " << MUON_MAX_NS_STEPS << "]"; err = s.str();
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (dtype != MUON_F32 && dtype != MUON_BF16) { err = "unknown dtype"; return MUON_ERR_INVALID_ARGUMENT; }
  return MUON_OK;
}

int check_ptr(const void* p, const char* what, int index, std::string& err) {
  if (!p) {
    std::ostringstream s; s << what << "[" << index << "] is NULL"; err = s.str();
    return MUON_ERR_INVALID_ARGUMENT;
  }
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) {
    std::ostringstream s; s << what << "[" << index << "] is not 16-byte aligned"; err = s.str();
    return MUON_ERR_MISALIGNED;
  }
  return MUON_OK;
}

Range strided_range(const void* p, unsigned long long rows, unsigned long long row_bytes,
                    unsigned long long ld_bytes, const char* what, int index) {
  Range r;
  r.lo = (unsigned long long)reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + (rows > 0 ? (rows - 1) * ld_bytes + row_bytes : 0);
  r.what = what;
  r.index = index;
  r.rows = rows;
  r.row_bytes = row_bytes;
  r.ld_bytes = ld_bytes;
  return r;
}

namespace {

// Whether two blocks with intersecting spans share a byte; a.lo <= b.lo.
// With equal strides L, b's rows sit at offset d = q L + rr in a's frame:
// b row k covers bytes [rr, rr + wb) of a's row q + k, wrapping into row
// q + k + 1 when rr + wb > L.
bool blocks_overlap(const Range& a, const Range& b) {
  const unsigned long long L = a.ld_bytes;
  if (L != b.ld_bytes || L == 0 || a.row_bytes > L || b.row_bytes > L) return true;
  const unsigned long long d = b.lo - a.lo, q = d / L, rr = d % L;
  if (rr < a.row_bytes && q < a.rows) return true;                 // b rows q.. on a's columns
  if (rr + b.row_bytes > L && q + 1 < a.rows) return true;         // wrapped part, a's rows q+1..
  return false;
}

}  // namespace

int check_no_overlap(std::vector<Range>& r, std::string& err) {
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 0; i < r.size(); ++i) {
    for (size_t j = i + 1; j < r.size() && r[j].lo < r[i].hi; ++j) {
      if (r[i].hi > r[i].lo && r[j].hi > r[j].lo && blocks_overlap(r[i], r[j])) {
        std::ostringstream s;
        s << r[i].what << "[" << r[i].index << "] overlaps " << r[j].what << "[" << r[j].index << "]";
        err = s.str();
        return MUON_ERR_INVALID_ARGUMENT;
      }
    }
  }
  return MUON_OK;
}

}  // namespace muon
