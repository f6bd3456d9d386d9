// Host side of the AReA library: argument validation, the integer schedule
// (pooling ramp, window shrink, base tiling, boundary shift), workspace
// sizing and the C entry points that enqueue the kernels.
#include <cmath>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "area_internal.h"

namespace area {

static thread_local std::string g_last_error;
static thread_local AttnEvents g_attn_events;

AttnEvents& attn_events() { return g_attn_events; }

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a < 0 ? -a : a;
}

int nearest_common_divisor(int a, int b, int lo, long long num, long long den) {
  int g = gcd_int(a, b);
  int best = -1;
  long long bestd = 0;
  for (int d = lo < 1 ? 1 : lo; d <= g; ++d) {
    if (g % d) continue;
    long long dist = (long long)d * den - num;
    if (dist < 0) dist = -dist;
    if (best < 0 || dist < bestd || (dist == bestd && d > best)) {
      best = d;
      bestd = dist;
    }
  }
  return best;
}

// READING R5 (blog "Las dos fases de AReA", Fase I; ai.info summary,
// Methodology, Phase I: f = 4 at 4096^2 maps the 256x256 grid to the native
// 64x64): the common divisor >= f_min nearest to the larger grid/native
// ratio, compared as exact fractions, ties to the larger divisor.
int derive_f0(const area_problem& p) {
  long long num, den;
  if ((long long)p.Gh * p.native_w >= (long long)p.Gw * p.native_h) {
    num = p.Gh;
    den = p.native_h;
  } else {
    num = p.Gw;
    den = p.native_w;
  }
  return nearest_common_divisor(p.Gh, p.Gw, p.f_min, num, den);
}

// READING R4: x_t = f0 + (f_min - f0) t / (P - 1), snapped to the nearest
// common divisor >= f_min (ties to the larger), in exact integers.
int ramp_factor(const area_problem& p, int f0, int t) {
  int P = p.p1_steps;
  if (P <= 1) return nearest_common_divisor(p.Gh, p.Gw, p.f_min, f0, 1);
  long long den = P - 1;
  long long num = (long long)f0 * den + (long long)(p.f_min - f0) * t;
  return nearest_common_divisor(p.Gh, p.Gw, p.f_min, num, den);
}

// READING R8 (ai.info summary, Phase II: evenly spaced base tiling):
// n = ceil(G / w) windows (1 if w >= G), b_i = round_half_up(i (G-w)/(n-1)).
void base_starts(int G, int w, std::vector<int>& out) {
  out.clear();
  if (w >= G) {
    out.push_back(0);
    return;
  }
  int n = (G + w - 1) / w;
  for (int i = 0; i < n; ++i)
    out.push_back((int)((2LL * i * (G - w) + (n - 1)) / (2LL * (n - 1))));
}

static int64_t axis_count(int G, int w) { return w >= G ? 1 : (G + w - 1) / w; }

// READING R7 (ai.info summary, Methodology, Phase II; blog, Fase II: the
// first window is the biggest whose windowed attention costs less than one
// pass of full attention, near 70% of the longer side): with
// p.w_start == 0, the largest even w in [w_min, max(Gh, Gw)] whose base
// tiling, each window attending to itself, has fewer (query, key) pairs than
// full attention: n_y n_x (min(w,Gh) min(w,Gw))^2 < (Gh Gw)^2, compared in
// 128-bit integers; w_min when nothing larger qualifies.
int w_start_of(const area_problem& p) {
  if (p.w_start > 0) return p.w_start;
  const unsigned __int128 N = (unsigned __int128)p.Gh * p.Gw;
  int best = p.w_min;
  for (int w = p.w_min; w <= std::max(p.Gh, p.Gw); ++w) {
    if (w % 2) continue;
    const unsigned __int128 area = (unsigned __int128)std::min(w, p.Gh) * std::min(w, p.Gw);
    const unsigned __int128 n = (unsigned __int128)axis_count(p.Gh, w) * axis_count(p.Gw, w);
    if (n * area * area < N * N) best = w;
  }
  return best;
}

// READING R6 (ai.info summary, Methodology, Phase II: geometric shrink from
// w_start to w_min): r_t = w_start (w_min / w_start)^(t / (S - 1)) in
// float64, then the nearest even integer, ties up.
int window_side(const area_problem& p, int t) {
  int S = p.p2_steps;
  const int w0 = w_start_of(p);
  double r;
  if (S <= 1) {
    r = (double)w0;
  } else {
    double ratio = (double)p.w_min / (double)w0;
    double e = (double)t / (double)(S - 1);
    r = (double)w0 * std::pow(ratio, e);
  }
  return 2 * (int)std::floor(r / 2.0 + 0.5);
}

// READING R19 (ai.info summary, Phase II; blog, Fase II: each window of side
// w gains (rho w)^2 bridge tokens, rho = 0.5): with bridge_rho_num > 0 the
// step's bridge has round_half_up(rho w_t)^2 tokens, else bridge_k.
int bridge_size(const area_problem& p, int w) {
  if (p.bridge_rho_num <= 0) return p.bridge_k;
  const long long side = (2LL * p.bridge_rho_num * w + p.bridge_rho_den) / (2LL * p.bridge_rho_den);
  return (int)std::min<long long>(side * side, 1LL << 30);
}

// SplitMix64 (Steele, Lea, Flood 2014): k-th output from state `seed`.
uint64_t splitmix64(uint64_t seed, uint64_t k) {
  uint64_t z = seed + k * 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

// READING R9 (blog, Fase II and the tunables list: the seed drives the
// border jitter): one shift per (step, axis) in [-J, J], J = half the
// smallest overlap of neighbouring windows, applied to interior windows.
int jitter_offset(const std::vector<int>& b, int L, uint64_t seed, int t, int axis) {
  int n = (int)b.size();
  if (n <= 2) return 0;
  int gap = 0;
  for (int i = 0; i + 1 < n; ++i) gap = std::max(gap, b[i + 1] - b[i]);
  int ov = L - gap;
  int J = ov > 0 ? ov / 2 : 0;
  if (J == 0) return 0;
  uint64_t r = splitmix64(seed, 2ULL * (uint64_t)t + (uint64_t)axis + 1ULL);
  return (int)(r % (uint64_t)(2 * J + 1)) - J;
}

bool axis_tiling(int G, int w, uint64_t seed, int t, int axis, AxisTiling& out) {
  std::vector<int> b;
  base_starts(G, w, b);
  if ((int)b.size() > kMaxAxisWindows) return false;
  out.n = (int)b.size();
  out.L = w < G ? w : G;
  out.jitter = jitter_offset(b, out.L, seed, t, axis);
  for (int i = 0; i < out.n; ++i) {
    out.start[i] = b[i] + ((i > 0 && i < out.n - 1) ? out.jitter : 0);
    if (out.start[i] < 0 || out.start[i] + out.L > G) return false;  // never: the shift keeps windows inside
  }
  return true;
}

// READING R13 (ai.info summary, Phase II: bridge tokens are spread over the
// image): one token per cell of an r_h x r_w = R grid.  Among the factor
// pairs with r_h <= Gh and r_w <= Gw the cells, (Gh / r_h) x (Gw / r_w)
// tokens, are the most nearly square: elongation max(Gh r_w, Gw r_h) /
// min(Gh r_w, Gw r_h), compared as exact 128-bit cross products; equal
// elongations go to the smaller r_h.  false when no pair fits.
bool bridge_cells(int R, int Gh, int Gw, int& rh, int& rw) {
  if (R < 1) return false;
  bool found = false;
  unsigned long long best_hi = 0, best_lo = 1;
  auto consider = [&](long long h, long long w) {
    if (h > Gh || w > Gw) return;
    const unsigned long long a = (unsigned long long)Gh * w, b = (unsigned long long)Gw * h;
    const unsigned long long hi = a > b ? a : b, lo = a > b ? b : a;
    const unsigned __int128 l = (unsigned __int128)hi * best_lo, r = (unsigned __int128)best_hi * lo;
    if (!found || l < r || (l == r && h < rh)) {
      found = true;
      best_hi = hi;
      best_lo = lo;
      rh = (int)h;
      rw = (int)w;
    }
  };
  for (long long d = 1; d * d <= R; ++d) {
    if (R % d) continue;
    consider(d, R / d);
    consider(R / d, d);
  }
  return found;
}

// README canvas rules: at or below native the original attention is kept.
bool canvas_gated(const area_problem& p) { return p.Gh <= p.native_h && p.Gw <= p.native_w; }

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int window_step(const area_problem& p, int step, WindowStepInfo& out) {
  if (canvas_gated(p)) return fail(AREA_E_INVALID, "canvas at or below native: no window steps");
  int t = step - p.p1_steps;
  if (step < 0 || t < 0 || t >= p.p2_steps)
    return fail(AREA_E_INVALID, "step " + std::to_string(step) + " is not a Phase II step");
  out.t = t;
  out.w = window_side(p, t);
  if (!axis_tiling(p.Gh, out.w, p.seed, t, 0, out.ty) ||
      !axis_tiling(p.Gw, out.w, p.seed, t, 1, out.tx))
    return fail(AREA_E_UNSUPPORTED, "more than 64 base windows per axis, or a window outside the grid");
  int64_t nb = (int64_t)out.ty.n * out.tx.n;
  int64_t Ly = out.ty.L, Lx = out.tx.L;
  out.q_total = nb * Ly * Lx;
  int64_t h1 = Ly / 2, w1 = Lx / 2;
  int64_t unsplit = ceil_div(Ly * Lx, kAttnBM);
  int64_t split = ceil_div(h1 * w1, kAttnBM) + ceil_div(h1 * (Lx - w1), kAttnBM) +
                  ceil_div((Ly - h1) * w1, kAttnBM) + ceil_div((Ly - h1) * (Lx - w1), kAttnBM);
  out.max_items = nb * (unsplit > split ? unsplit : split);
  // gathered key tiles: Halo rectangle (clipped to the grid, widest Halo) +
  // all R bridge slots per window, rounded up to 64 keys
  out.R = bridge_size(p, out.w);
  int64_t R = out.R;
  int64_t hw = p.halo_max > 0 ? p.halo_max : p.halo;
  int64_t kh = std::min<int64_t>(Ly + 2 * hw, p.Gh), kw = std::min<int64_t>(Lx + 2 * hw, p.Gw);
  int64_t qh = std::min<int64_t>(Ly - h1 + 2 * hw, p.Gh), qw = std::min<int64_t>(Lx - w1 + 2 * hw, p.Gw);
  int64_t g_unsplit = ceil_div(kh * kw + R + p.T, kAttnBN);
  int64_t g_split = 4 * ceil_div(qh * qw + R + p.T, kAttnBN);
  out.max_gtiles = nb * (g_unsplit > g_split ? g_unsplit : g_split);
  return AREA_OK;
}

static std::string pstr(const char* what, long long v) { return std::string(what) + "=" + std::to_string(v); }

static int validate(const area_problem* pp) {
  if (!pp) return fail(AREA_E_INVALID, "problem is NULL");
  const area_problem& p = *pp;
  if (p.B < 1 || p.H < 1 || p.Gh < 1 || p.Gw < 1 || p.native_h < 1 || p.native_w < 1)
    return fail(AREA_E_INVALID, "B, H, Gh, Gw, native_h, native_w must be positive");
  if (p.D != 64 && p.D != 128) return fail(AREA_E_UNSUPPORTED, pstr("head dim D must be 64 or 128, D", p.D));
  if (p.T < 0 || p.T > (1 << 20)) return fail(AREA_E_INVALID, pstr("text tokens must be in 0 .. 2^20, T", p.T));
  if (!(p.rope_theta > 0.0f) || !std::isfinite(p.rope_theta))
    return fail(AREA_E_INVALID, "rope_theta must be positive and finite");
  if (p.p1_steps < 0 || p.p2_steps < 0) return fail(AREA_E_INVALID, "step counts must be >= 0");
  if (p.pool_mode < AREA_POOL_MEAN || p.pool_mode > AREA_POOL_RANDOM)
    return fail(AREA_E_INVALID, pstr("pool_mode", p.pool_mode));
  if (p.f_min < 1 || p.f0 < 0) return fail(AREA_E_INVALID, "f_min must be >= 1 and f0 >= 0");
  if (p.halo < 0 || p.bridge_k < 0 || p.halo_max < 0)
    return fail(AREA_E_INVALID, "halo, halo_max and bridge_k must be >= 0");
  if (p.bridge_rho_num < 0 || (p.bridge_rho_num > 0 && p.bridge_rho_den <= 0))
    return fail(AREA_E_INVALID, "bridge_rho_num >= 0, and bridge_rho_den > 0 when it is used");
  if (p.split_den <= 0 || p.split_num < 0) return fail(AREA_E_INVALID, "split_num >= 0, split_den > 0");
  long long N = (long long)p.Gh * p.Gw;
  if (N + p.T > (1LL << 30) || (long long)p.B * p.H * (N + p.T) * p.D > (1LL << 40))
    return fail(AREA_E_UNSUPPORTED, "problem too large");
  // the (cos, sin) tables hold max(Gh, Gw) x D/4 entries indexed in 32 bits
  if (p.Gh > kMaxGridSide || p.Gw > kMaxGridSide)
    return fail(AREA_E_UNSUPPORTED, pstr("grid sides must be at most 65536, max side", std::max(p.Gh, p.Gw)));
  if (p.Gh % 2 || p.Gw % 2) return fail(AREA_E_SHAPE, "both grid sides must be even");
  if (canvas_gated(p)) return AREA_OK;  // full attention only; the knobs below are unused
  int fl = p.f_min > 2 ? p.f_min : 2;
  if (gcd_int(p.Gh, p.Gw) < fl)
    return fail(AREA_E_SHAPE, "grid sides share no factor >= max(2, f_min) (README canvas rules)");
  if (p.f0 > 0 && (p.Gh % p.f0 || p.Gw % p.f0 || p.f0 < p.f_min))
    return fail(AREA_E_SHAPE, pstr("f0 must be a common grid divisor >= f_min, f0", p.f0));
  if (p.f0 == 0 && derive_f0(p) < 0) return fail(AREA_E_SHAPE, "no pooling factor fits the grid");
  if (p.p2_steps > 0) {
    if (p.w_min < 2 || p.w_min % 2 || (p.w_start != 0 && (p.w_start < p.w_min || p.w_start % 2)))
      return fail(AREA_E_SHAPE, "window sides must be even with 2 <= w_min <= w_start (w_start 0: derived)");
    int nmax_y = (p.Gh + p.w_min - 1) / p.w_min, nmax_x = (p.Gw + p.w_min - 1) / p.w_min;
    if (nmax_y > kMaxAxisWindows || nmax_x > kMaxAxisWindows)
      return fail(AREA_E_UNSUPPORTED, "w_min gives more than 64 base windows per axis");
    for (int t = 0; t < p.p2_steps; ++t) {
      const int R = bridge_size(p, window_side(p, t));
      if (R <= 0) continue;
      int rh, rw;
      if (!bridge_cells(R, p.Gh, p.Gw, rh, rw))
        return fail(AREA_E_SHAPE, pstr("bridge cells do not fit the grid, R", R));
      if (rw > kBridgeSortMax) return fail(AREA_E_UNSUPPORTED, pstr("bridge cell rows above 4096 cells, R", R));
    }
  }
  return AREA_OK;
}

static int64_t BH_of(const area_problem& p) { return (int64_t)p.B * p.H; }
static int64_t N_of(const area_problem& p) { return (int64_t)p.Gh * p.Gw; }
static int64_t L_of(const area_problem& p) { return (int64_t)p.T + N_of(p); }  // rows per sequence
static size_t tok_bytes(const area_problem& p) { return (size_t)BH_of(p) * L_of(p) * p.D * 2; }

// Regions of the dense-attention workspace (full attention, the text pass
// and coarse attention; M = T + Gh*Gw key rows per (batch, head) covers
// every pooling factor down to f = 1): fp16 key rows, fp16 V^T tiles, the
// (cos, sin) tables, per-tile exponents of K and V, per-(batch, head) range
// flags.
struct DenseLayout {
  size_t kr, vt, tab, kexp, vexp, flags, total;
};

static DenseLayout dense_layout(const area_problem& p) {
  const int64_t BH = BH_of(p);
  const int M = (int)L_of(p);
  DenseLayout l;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align_up(bytes);
    return at;
  };
  l.kr = take(tok_bytes(p));
  l.vt = take(vt_bytes(BH, M, p.D));
  l.tab = take(rope_table_bytes(p.Gh, p.Gw, p.D));
  l.kexp = take(tile_exp_bytes(BH, M));
  l.vexp = take(tile_exp_bytes(BH, M));
  l.flags = take(range_words(BH, BH * (((int64_t)M + kAttnBM - 1) / kAttnBM)) * sizeof(int));
  l.total = off;
  return l;
}

struct WindowMax {
  int64_t q_total = 0, max_items = 0, max_gtiles = 0;
  int max_windows = 0, n_base = 0, max_R = 0;
};

static WindowMax window_max(const area_problem& p) {
  WindowMax m;
  for (int t = 0; t < p.p2_steps; ++t) {
    WindowStepInfo wi;
    if (window_step(p, p.p1_steps + t, wi) != AREA_OK) continue;
    int nb = wi.ty.n * wi.tx.n;
    m.q_total = std::max<int64_t>(m.q_total, wi.q_total);
    m.max_items = std::max<int64_t>(m.max_items, wi.max_items);
    m.max_gtiles = std::max<int64_t>(m.max_gtiles, wi.max_gtiles);
    m.max_windows = std::max(m.max_windows, 4 * nb);
    m.n_base = std::max(m.n_base, nb);
    m.max_R = std::max(m.max_R, wi.R);
  }
  return m;
}

// Regions of the windowed-attention workspace, in order.
struct WindowLayout {
  size_t rope, slots, items, kg, vg, blist, bcount, kexp, vexp, flags, total;
};

static WindowLayout window_layout(const area_problem& p) {
  WindowMax m = window_max(p);
  int64_t BH = BH_of(p);
  WindowLayout l;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align_up(bytes);
    return at;
  };
  l.rope = take(rope_table_bytes(p.Gh, p.Gw, p.D));
  l.slots = take((size_t)m.q_total * BH * p.D * 4);
  l.items = take(window_items_ws_bytes(m.max_windows, m.max_items, m.n_base, m.max_gtiles));
  l.kg = take((size_t)BH * m.max_gtiles * kAttnBN * p.D * 2);
  l.vg = take((size_t)BH * m.max_gtiles * kAttnBN * p.D * 2);
  l.blist = take((size_t)m.max_windows * BH * std::max(m.max_R, 1) * 4);
  l.bcount = take((size_t)m.max_windows * BH * 4);
  l.kexp = take((size_t)BH * m.max_gtiles * sizeof(int));
  l.vexp = take((size_t)BH * m.max_gtiles * sizeof(int));
  l.flags = take(range_words(BH, BH * m.max_items) * sizeof(int));
  l.total = off;
  return l;
}

// Intermediates of area_attn_step, carved from its workspace: coarse steps
// hold the pooled K and V (largest for the smallest factor of the ramp);
// window steps hold the energy map, plan, weight sums and bridge indices.
// Each phase's own workspace follows its intermediates.
struct StepLayout {
  size_t kp = 0, vp = 0, coarse_ws = 0;                          // coarse
  size_t energy = 0, energy_q = 0, plan = 0, wsum = 0, bridge = 0, window_ws = 0;  // window
  size_t total = 0;
};

static size_t workspace_bytes(const area_problem& p, int op);

static StepLayout step_layout(const area_problem& p) {
  StepLayout l;
  const size_t N = (size_t)N_of(p), BH = (size_t)BH_of(p);
  if (canvas_gated(p)) {
    l.total = workspace_bytes(p, AREA_OP_FULL);
    return l;
  }
  size_t coarse = 0, window = 0;
  if (p.p1_steps > 0) {
    int f0 = p.f0 > 0 ? p.f0 : derive_f0(p);
    size_t M = 0;
    for (int s = 0; s < p.p1_steps; ++s) {
      int f = ramp_factor(p, f0, s);
      M = std::max(M, N / ((size_t)f * f));
    }
    const size_t pooled = align_up(BH * (M + p.T) * p.D * 4);  // fp32 pooled rows
    l.kp = 0;
    l.vp = pooled;
    l.coarse_ws = 2 * pooled;
    coarse = l.coarse_ws + std::max(workspace_bytes(p, AREA_OP_COARSE),
                                     p.T > 0 ? workspace_bytes(p, AREA_OP_FULL) : (size_t)0);
  }
  if (p.p2_steps > 0) {
    size_t o = 0;
    l.energy = o;
    o += align_up(N / 4 * 4);
    l.energy_q = o;
    o += align_up(N / 4 * 4);
    l.plan = o;
    o += align_up((AREA_PLAN_HEADER + (size_t)AREA_PLAN_REC * window_max(p).max_windows) * 4);
    l.wsum = o;
    o += align_up(N * 4);
    l.bridge = o;
    o += align_up(BH * std::max(window_max(p).max_R, 1) * 4);
    l.window_ws = o;
    window = o + std::max({workspace_bytes(p, AREA_OP_PLAN), workspace_bytes(p, AREA_OP_WINDOW),
                           p.T > 0 ? workspace_bytes(p, AREA_OP_FULL) : (size_t)0});
  }
  l.total = std::max(coarse, window);
  return l;
}

static size_t workspace_bytes(const area_problem& p, int op) {
  switch (op) {
    case AREA_OP_STEP:
      return step_layout(p).total;
    case AREA_OP_FULL:    // key rows, V^T tiles, (cos, sin) tables, tile exponents, flags
    case AREA_OP_COARSE:  // the same for the pooled keys and values
      return dense_layout(p).total;
    case AREA_OP_PLAN: {
      if (canvas_gated(p) || p.p2_steps == 0) return 0;
      WindowMax m = window_max(p);
      return align_up(plan_ws_bytes(m.n_base)) +
             align_up(bridge_ws_bytes(BH_of(p), (int)N_of(p), p.D, m.max_R));
    }
    case AREA_OP_WINDOW: {
      if (canvas_gated(p) || p.p2_steps == 0) return 0;
      return window_layout(p).total;
    }
    default:
      return 0;
  }
}

static int check_ws(const area_problem& p, int op, void* ws, size_t ws_bytes) {
  size_t need = workspace_bytes(p, op);
  if (need == 0) return AREA_OK;
  if (!ws) return fail(AREA_E_WORKSPACE, "workspace is NULL, need " + std::to_string(need) + " bytes");
  if (ws_bytes < need)
    return fail(AREA_E_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, need " +
                                      std::to_string(need));
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(AREA_E_WORKSPACE, "workspace must be 256-byte aligned");
  return AREA_OK;
}

// Dense attention of query rows q0 .. q0 + Nq - 1 over every key of the
// sequences (text and image, RoPE at native positions; text at (0, 0)) in a
// workspace of dense_layout: full attention (all rows) and the text pass
// (the T text rows).
static int dense_pass(const area_problem& p, char* b, const void* q, const void* k, const void* v, void* out, int q0,
                      int Nq, void* stream) {
  const int64_t BH = BH_of(p);
  const int L = (int)L_of(p);
  const DenseLayout l = dense_layout(p);
  int* kexp = (int*)(b + l.kexp);
  int* vexp = (int*)(b + l.vexp);
  int* flags = (int*)(b + l.flags);
  int rc = launch_rope_table(b + l.tab, p.Gh, p.Gw, p.D, p.rope_theta, 1.0f, flags, range_clear_words(BH), stream);
  if (rc) return rc;
  rc = launch_kv_tiles(k, v, b + l.tab, b + l.kr, b + l.vt, kexp, vexp, flags, BH, L, p.D, false, p.T, p.Gw, stream);
  if (rc) return rc;
  return launch_dense_attn(q, b + l.tab, p.T, p.Gh, p.Gw, b + l.kr, b + l.vt, kexp, vexp, flags, out, BH, Nq, q0, L,
                           L, p.D, stream);
}

}  // namespace area

using namespace area;

extern "C" {

int area_validate(const area_problem* p) { return validate(p); }

int area_f0(const area_problem* p) {
  int rc = validate(p);
  if (rc) return rc;
  if (canvas_gated(*p)) return 1;
  return p->f0 > 0 ? p->f0 : derive_f0(*p);
}

int area_step_info(const area_problem* p, int step, area_step* out) {
  int rc = validate(p);
  if (rc) return rc;
  if (!out) return fail(AREA_E_INVALID, "out is NULL");
  std::memset(out, 0, sizeof(*out));
  int total = p->p1_steps + p->p2_steps;
  if (step < 0 || step >= total) return fail(AREA_E_INVALID, "step out of range");
  if (canvas_gated(*p)) {
    out->phase = AREA_PHASE_FULL;
    return AREA_OK;
  }
  if (step < p->p1_steps) {
    int f0 = p->f0 > 0 ? p->f0 : derive_f0(*p);
    out->phase = AREA_PHASE_COARSE;
    out->f = ramp_factor(*p, f0, step);
    return AREA_OK;
  }
  WindowStepInfo wi;
  rc = window_step(*p, step, wi);
  if (rc) return rc;
  out->phase = AREA_PHASE_WINDOW;
  out->w = wi.w;
  out->ny = wi.ty.n;
  out->nx = wi.tx.n;
  out->jit_y = wi.ty.jitter;
  out->jit_x = wi.tx.jitter;
  out->max_windows = 4 * wi.ty.n * wi.tx.n;
  out->q_total = wi.q_total;
  out->R = wi.R;
  if (wi.R > 0) bridge_cells(wi.R, p->Gh, p->Gw, out->bridge_rh, out->bridge_rw);
  return AREA_OK;
}

int area_base_windows(const area_problem* p, int step, int32_t* out, int cap) {
  int rc = validate(p);
  if (rc) return rc;
  WindowStepInfo wi;
  rc = window_step(*p, step, wi);
  if (rc) return rc;
  int n = wi.ty.n * wi.tx.n;
  if (!out || cap < n) return fail(AREA_E_INVALID, "output array too small: need " + std::to_string(n));
  int k = 0;
  for (int i = 0; i < wi.ty.n; ++i)
    for (int j = 0; j < wi.tx.n; ++j) {
      out[4 * k + 0] = wi.ty.start[i];
      out[4 * k + 1] = wi.tx.start[j];
      out[4 * k + 2] = wi.ty.L;
      out[4 * k + 3] = wi.tx.L;
      ++k;
    }
  return n;
}

size_t area_workspace_bytes(const area_problem* p, int op) {
  if (validate(p)) return 0;
  return workspace_bytes(*p, op);
}

size_t area_plan_words(const area_problem* p) {
  if (validate(p) || canvas_gated(*p) || p->p2_steps == 0) return 0;
  WindowMax m = window_max(*p);
  return AREA_PLAN_HEADER + (size_t)AREA_PLAN_REC * m.max_windows;
}

const char* area_strerror(int status) {
  switch (status) {
    case AREA_OK: return "ok";
    case AREA_E_INVALID: return "invalid argument";
    case AREA_E_SHAPE: return "inconsistent shape";
    case AREA_E_UNSUPPORTED: return "unsupported configuration";
    case AREA_E_WORKSPACE: return "workspace missing or too small";
    case AREA_E_HIP: return "HIP runtime failure";
    default: return "unknown status";
  }
}

const char* area_last_error(void) { return g_last_error.c_str(); }

int area_set_attn_events(void* ev_begin, void* ev_end) {
  if ((ev_begin == nullptr) != (ev_end == nullptr))
    return fail(AREA_E_INVALID, "pass both events or neither");
  g_attn_events.begin = ev_begin;
  g_attn_events.end = ev_end;
  return AREA_OK;
}

int area_phase1_steps_for_sigma(const double* sigmas, int n_steps, double sigma_star, int* p1_steps) {
  if (!p1_steps || (n_steps > 0 && !sigmas)) return fail(AREA_E_INVALID, "NULL sigmas or result pointer");
  if (n_steps < 0) return fail(AREA_E_INVALID, pstr("n_steps", n_steps));
  if (sigma_star != sigma_star) return fail(AREA_E_INVALID, "sigma_star is NaN");
  int n = 0;
  while (n < n_steps && sigmas[n] > sigma_star) ++n;
  *p1_steps = n;
  return AREA_OK;
}

int area_measure_mfma_peak(void* sink, double* tflops, void* stream) {
  if (!sink || !tflops) return fail(AREA_E_INVALID, "NULL sink or result pointer");
  return measure_mfma_peak(sink, tflops, stream);
}

int area_pool_kv(const area_problem* p, int f, const void* k, const void* v, void* kp, void* vp,
                 void* stream) {
  int rc = validate(p);
  if (rc) return rc;
  if (!k || !v || !kp || !vp) return fail(AREA_E_INVALID, "NULL tensor");
  if (f < 1 || p->Gh % f || p->Gw % f) return fail(AREA_E_SHAPE, pstr("f must divide both grid sides, f", f));
  return launch_pool(k, v, kp, vp, BH_of(*p), p->T, p->Gh, p->Gw, p->D, f, p->pool_mode, p->seed, p->rope_theta,
                     stream);
}

int area_coarse_attn(const area_problem* p, int f, const void* q, const void* kp, const void* vp,
                     void* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate(p);
  if (rc) return rc;
  if (!q || !kp || !vp || !out) return fail(AREA_E_INVALID, "NULL tensor");
  if (f < 1 || p->Gh % f || p->Gw % f) return fail(AREA_E_SHAPE, pstr("f must divide both grid sides, f", f));
  rc = check_ws(*p, AREA_OP_COARSE, ws, ws_bytes);
  if (rc) return rc;
  const int64_t BH = BH_of(*p);
  const int N = (int)N_of(*p);
  const int M = p->T + N / (f * f);  // text rows, then the pooled grid
  const DenseLayout l = dense_layout(*p);
  char* b = (char*)ws;
  int* kexp = (int*)(b + l.kexp);
  int* vexp = (int*)(b + l.vexp);
  int* flags = (int*)(b + l.flags);
  // queries turn at coarse-grid positions (row / f, column / f), as the keys
  rc = launch_rope_table(b + l.tab, p->Gh, p->Gw, p->D, p->rope_theta, (float)f, flags, range_clear_words(BH), stream);
  if (rc) return rc;
  rc = launch_kv_tiles(kp, vp, b + l.tab, b + l.kr, b + l.vt, kexp, vexp, flags, BH, M, p->D, true, p->T, p->Gw,
                       stream);
  if (rc) return rc;
  return launch_dense_attn(q, b + l.tab, p->T, p->Gh, p->Gw, b + l.kr, b + l.vt, kexp, vexp, flags, out, BH, N, p->T,
                           p->T + N, M, p->D, stream);
}

int area_full_attn(const area_problem* p, const void* q, const void* k, const void* v, void* out,
                   void* ws, size_t ws_bytes, void* stream) {
  int rc = validate(p);
  if (rc) return rc;
  if (!q || !k || !v || !out) return fail(AREA_E_INVALID, "NULL tensor");
  rc = check_ws(*p, AREA_OP_FULL, ws, ws_bytes);
  if (rc) return rc;
  return dense_pass(*p, (char*)ws, q, k, v, out, 0, (int)L_of(*p), stream);
}

}  // extern "C"

namespace area {



}  // namespace area

extern "C" {

int area_text_attn(const area_problem* p, const void* q, const void* k, const void* v, void* out, void* ws,
                   size_t ws_bytes, void* stream) {
  int rc = validate(p);
  if (rc) return rc;
  if (!q || !k || !v || !out) return fail(AREA_E_INVALID, "NULL tensor");
  if (p->T == 0) return AREA_OK;
  rc = check_ws(*p, AREA_OP_FULL, ws, ws_bytes);
  if (rc) return rc;
  return dense_pass(*p, (char*)ws, q, k, v, out, 0, p->T, stream);
}

int area_dwt_detail(const area_problem* p, int C, const float* latent, float* energy,
                    int32_t* energy_q, void* stream) {
  int rc = validate(p);
  if (rc) return rc;
  if (C < 1) return fail(AREA_E_INVALID, "C must be >= 1");
  if (!latent || !energy || !energy_q) return fail(AREA_E_INVALID, "NULL tensor");
  return launch_dwt(latent, energy, energy_q, C, p->Gh, p->Gw, stream);
}

int area_window_plan(const area_problem* p, int step, const int32_t* energy_q, const void* k,
                     int32_t* plan, int32_t* wsum, int32_t* bridge_idx, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc = validate(p);
  if (rc) return rc;
  WindowStepInfo wi;
  rc = window_step(*p, step, wi);
  if (rc) return rc;
  if (!plan || !wsum) return fail(AREA_E_INVALID, "NULL plan or wsum");
  bool use_bridge = wi.R > 0 && k != nullptr;
  if (use_bridge && !bridge_idx) return fail(AREA_E_INVALID, "bridge_idx is NULL");
  rc = check_ws(*p, AREA_OP_PLAN, ws, ws_bytes);
  if (rc) return rc;
  PlanArgs a;
  std::memset(&a, 0, sizeof(a));
  a.Gh = p->Gh;
  a.Gw = p->Gw;
  a.halo = p->halo_max > 0 ? p->halo_max : p->halo;
  a.halo_max = p->halo_max;
  a.seed = p->seed;
  a.R = use_bridge ? wi.R : 0;
  a.split_num = p->split_num;
  a.split_den = energy_q ? p->split_den : 0;  // 0: never split
  a.t = wi.t;
  a.w = wi.w;
  a.ny = wi.ty.n;
  a.nx = wi.tx.n;
  a.jit_y = wi.ty.jitter;
  a.jit_x = wi.tx.jitter;
  a.Ly = wi.ty.L;
  a.Lx = wi.tx.L;
  for (int i = 0; i < a.ny; ++i) a.ys[i] = wi.ty.start[i];
  for (int i = 0; i < a.nx; ++i) a.xs[i] = wi.tx.start[i];
  WindowMax m = window_max(*p);
  char* wsb = (char*)ws;
  rc = launch_plan(a, energy_q, plan, wsum, wsb, stream);
  if (rc) return rc;
  if (use_bridge) {
    int rh, rw;
    bridge_cells(wi.R, p->Gh, p->Gw, rh, rw);
    rc = launch_bridge(k, bridge_idx, BH_of(*p), p->T, p->Gh, p->Gw, p->D, wi.R, rh, rw,
                       wsb + align_up(plan_ws_bytes(m.n_base)), stream);
  }
  return rc;
}

int area_window_attn(const area_problem* p, int step, const int32_t* plan, const int32_t* wsum,
                     const int32_t* bridge_idx, const void* q, const void* k, const void* v,
                     void* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate(p);
  if (rc) return rc;
  WindowStepInfo wi;
  rc = window_step(*p, step, wi);
  if (rc) return rc;
  if (!plan || !wsum || !q || !k || !v || !out) return fail(AREA_E_INVALID, "NULL tensor");
  rc = check_ws(*p, AREA_OP_WINDOW, ws, ws_bytes);
  if (rc) return rc;
  WindowAttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.Gh = p->Gh;
  a.Gw = p->Gw;
  a.D = p->D;
  a.R = (bridge_idx && wi.R > 0) ? wi.R : 0;
  a.T = p->T;
  a.BH = BH_of(*p);
  a.max_windows = 4 * wi.ty.n * wi.tx.n;
  a.max_items = wi.max_items;
  a.max_gtiles = wi.max_gtiles;
  a.ny = wi.ty.n;
  a.nx = wi.tx.n;
  a.Ly = wi.ty.L;
  a.Lx = wi.tx.L;
  for (int i = 0; i < a.ny; ++i) a.ys[i] = wi.ty.start[i];
  for (int i = 0; i < a.nx; ++i) a.xs[i] = wi.tx.start[i];
  WindowLayout l = window_layout(*p);
  char* base = (char*)ws;
  WindowWs w;
  w.items = base + l.items;
  w.slots = (float*)(base + l.slots);
  w.kg = base + l.kg;
  w.vg = base + l.vg;
  w.blist = (int*)(base + l.blist);
  w.bcount = (int*)(base + l.bcount);
  w.kexp = (int*)(base + l.kexp);
  w.vexp = (int*)(base + l.vexp);
  w.flags = (int*)(base + l.flags);
  rc = launch_rope_table(base + l.rope, p->Gh, p->Gw, p->D, p->rope_theta, 1.0f, w.flags, range_clear_words(BH_of(*p)), stream);
  if (rc) return rc;
  return launch_window_attn(a, plan, wsum, a.R ? bridge_idx : nullptr, q, k, v, base + l.rope, out, w, stream);
}

int area_attn_step(const area_problem* p, int step, int C, const float* latent, const void* q,
                   const void* k, const void* v, void* out, void* ws, size_t ws_bytes, void* stream) {
  area_step st;
  int rc = area_step_info(p, step, &st);
  if (rc) return rc;
  if (!q || !k || !v || !out) return fail(AREA_E_INVALID, "NULL tensor");
  if (latent && C < 1) return fail(AREA_E_INVALID, "C must be >= 1");
  rc = check_ws(*p, AREA_OP_STEP, ws, ws_bytes);
  if (rc) return rc;
  const StepLayout l = step_layout(*p);
  char* base = (char*)ws;
  switch (st.phase) {
    case AREA_PHASE_FULL:
      return area_full_attn(p, q, k, v, out, ws, ws_bytes, stream);
    case AREA_PHASE_COARSE: {
      void* kp = base + l.kp;
      void* vp = base + l.vp;
      rc = area_pool_kv(p, st.f, k, v, kp, vp, stream);
      if (rc) return rc;
      rc = area_coarse_attn(p, st.f, q, kp, vp, out, base + l.coarse_ws, ws_bytes - l.coarse_ws, stream);
      if (rc) return rc;
      return area_text_attn(p, q, k, v, out, base + l.coarse_ws, ws_bytes - l.coarse_ws, stream);
    }
    default: {
      float* energy = (float*)(base + l.energy);
      int32_t* energy_q = (int32_t*)(base + l.energy_q);
      int32_t* plan = (int32_t*)(base + l.plan);
      int32_t* wsum = (int32_t*)(base + l.wsum);
      int32_t* bridge = st.R > 0 ? (int32_t*)(base + l.bridge) : nullptr;
      if (latent) {
        rc = area_dwt_detail(p, C, latent, energy, energy_q, stream);
        if (rc) return rc;
      }
      rc = area_window_plan(p, step, latent ? energy_q : nullptr, k, plan, wsum, bridge, base + l.window_ws,
                            ws_bytes - l.window_ws, stream);
      if (rc) return rc;
      rc = area_window_attn(p, step, plan, wsum, bridge, q, k, v, out, base + l.window_ws,
                            ws_bytes - l.window_ws, stream);
      if (rc || p->T == 0) return rc;
      return dense_pass(*p, base + l.window_ws, q, k, v, out, 0, p->T, stream);
    }
  }
}

}  // extern "C"
