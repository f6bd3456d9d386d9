// Host-only stand-in for the kernel launchers of libarea, for the sanitizer
// build of the library's host code (area_host.cpp + area_sizes.cpp, compiled
// with g++ -fsanitize=address,undefined; see tests/test_host_sanitized.py).
//
// No kernel runs.  Each launcher instead touches, in host memory, every
// buffer region the real kernels read or write, with the extents the kernels
// derive from the same arguments: reads scan the bytes, writes fill them.
// The caller passes host buffers in place of device memory, so AddressSanitizer
// reports any region that runs past its allocation.  A launcher also checks
// that the regions it writes overlap none of the other regions it was given
// (a workspace layout that carves two regions over each other fails here).
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "area_internal.h"

namespace area {

namespace {

struct Region {
  const char* what;
  const char* p;
  size_t bytes;
  bool write;
};

volatile unsigned char g_sink;

int check(std::vector<Region>& rs, const char* call) {
  for (auto& r : rs) {
    if (r.bytes == 0) continue;
    if (!r.p) return fail(AREA_E_HIP, std::string(call) + ": NULL region " + r.what);
    if (r.write) {
      std::memset((void*)r.p, 0, r.bytes);
    } else {
      unsigned char acc = 0;
      for (size_t i = 0; i < r.bytes; i += 64) acc ^= (unsigned char)r.p[i];
      acc ^= (unsigned char)r.p[r.bytes - 1];
      g_sink = acc;
    }
  }
  for (size_t i = 0; i < rs.size(); ++i) {
    if (!rs[i].write || rs[i].bytes == 0) continue;
    for (size_t j = 0; j < rs.size(); ++j) {
      if (j == i || rs[j].bytes == 0) continue;
      const char *a0 = rs[i].p, *a1 = rs[i].p + rs[i].bytes, *b0 = rs[j].p, *b1 = rs[j].p + rs[j].bytes;
      if (a0 < b1 && b0 < a1)
        return fail(AREA_E_HIP, std::string(call) + ": written region " + rs[i].what + " overlaps " + rs[j].what);
    }
  }
  return AREA_OK;
}

size_t words_of_range(int64_t BH, int64_t work) { return range_words(BH, work) * sizeof(int); }

}  // namespace

int launch_rope_table(void* tab, int Gh, int Gw, int D, float theta, float div, int* flags, int64_t n_flags,
                      stream_t) {
  std::vector<Region> r = {{"rope table", (const char*)tab, rope_table_bytes(Gh, Gw, D), true},
                           {"range flags", (const char*)flags, (size_t)n_flags * sizeof(int), true}};
  return check(r, "launch_rope_table");
}

int launch_pool(const void* k, const void* v, void* kp, void* vp, int64_t BH, int T, int Gh, int Gw, int D, int f,
                int, unsigned long long, float, stream_t) {
  const size_t in = (size_t)BH * ((size_t)T + (size_t)Gh * Gw) * D * 2;
  const size_t out = (size_t)BH * ((size_t)T + (size_t)(Gh / f) * (Gw / f)) * D * 4;
  std::vector<Region> r = {{"k", (const char*)k, in, false}, {"v", (const char*)v, in, false},
                           {"kp", (const char*)kp, out, true}, {"vp", (const char*)vp, out, true}};
  return check(r, "launch_pool");
}

int launch_dwt(const float* latent, float* energy, int32_t* energy_q, int C, int Gh, int Gw, stream_t) {
  const size_t cells = (size_t)(Gh / 2) * (Gw / 2);
  std::vector<Region> r = {{"latent", (const char*)latent, (size_t)C * Gh * Gw * 4, false},
                           {"energy", (const char*)energy, cells * 4, true},
                           {"energy_q", (const char*)energy_q, cells * 4, true}};
  return check(r, "launch_dwt");
}

int launch_plan(const PlanArgs& a, const int32_t* energy_q, int32_t* plan, int32_t* wsum, void* ws, stream_t) {
  const int nb = a.ny * a.nx;
  if (a.ny < 1 || a.nx < 1 || a.ny > kMaxAxisWindows || a.nx > kMaxAxisWindows)
    return fail(AREA_E_HIP, "launch_plan: base window count out of range");
  for (int i = 0; i < a.ny; ++i)
    if (a.ys[i] < 0 || a.ys[i] + a.Ly > a.Gh) return fail(AREA_E_HIP, "launch_plan: window row outside the grid");
  for (int i = 0; i < a.nx; ++i)
    if (a.xs[i] < 0 || a.xs[i] + a.Lx > a.Gw) return fail(AREA_E_HIP, "launch_plan: window column outside the grid");
  std::vector<Region> r = {
      {"energy_q", (const char*)energy_q, a.split_den > 0 ? (size_t)(a.Gh / 2) * (a.Gw / 2) * 4 : 0, false},
      {"plan", (const char*)plan, (AREA_PLAN_HEADER + (size_t)AREA_PLAN_REC * 4 * nb) * 4, true},
      {"wsum", (const char*)wsum, (size_t)a.Gh * a.Gw * 4, true},
      {"plan workspace", (const char*)ws, plan_ws_bytes(nb), true}};
  return check(r, "launch_plan");
}

int launch_bridge(const void* k, int32_t* idx, int64_t BH, int T, int Gh, int Gw, int D, int R, int rh, int rw,
                  void* ws, stream_t) {
  if (rh < 1 || rw < 1 || (int64_t)rh * rw != R || rh > Gh || rw > Gw)
    return fail(AREA_E_HIP, "launch_bridge: cell grid inconsistent with R and the grid");
  std::vector<Region> r = {{"k", (const char*)k, (size_t)BH * ((size_t)T + (size_t)Gh * Gw) * D * 2, false},
                           {"bridge_idx", (const char*)idx, (size_t)BH * R * 4, true},
                           {"bridge workspace", (const char*)ws, bridge_ws_bytes(BH, Gh * Gw, D, R), true}};
  return check(r, "launch_bridge");
}

int launch_kv_tiles(const void* k, const void* v, const void* rope, void* kr, void* vt, int* kexp, int* vexp,
                    int* flags, int64_t BH, int M, int D, bool f32_in, int, int, stream_t) {
  const size_t in = (size_t)BH * M * D * (f32_in ? 4 : 2);
  std::vector<Region> r = {{"k", (const char*)k, in, false},
                           {"v", (const char*)v, in, false},
                           {"rope table", (const char*)rope, 8, false},
                           {"key rows", (const char*)kr, (size_t)BH * M * D * 2, true},
                           {"V^T tiles", (const char*)vt, vt_bytes(BH, M, D), true},
                           {"K exponents", (const char*)kexp, tile_exp_bytes(BH, M), true},
                           {"V exponents", (const char*)vexp, tile_exp_bytes(BH, M), true},
                           {"range flags", (const char*)flags, (size_t)BH * sizeof(int), true}};
  return check(r, "launch_kv_tiles");
}

int launch_dense_attn(const void* q, const void* rope, int, int Gh, int Gw, const void* k_rot, const void* vt,
                      const int* kexp, const int* vexp, int* flags, void* out, int64_t BH, int Nq, int q0, int q_rows,
                      int Nk, int D, stream_t) {
  if (q0 < 0 || Nq < 0 || q0 + Nq > q_rows) return fail(AREA_E_HIP, "launch_dense_attn: query rows outside the sequence");
  const int64_t work = BH * (((int64_t)Nq + kAttnBM - 1) / kAttnBM);
  std::vector<Region> r = {{"q", (const char*)q, (size_t)BH * q_rows * D * 2, false},
                           {"rope table", (const char*)rope, rope_table_bytes(Gh, Gw, D), false},
                           {"key rows", (const char*)k_rot, (size_t)BH * Nk * D * 2, false},
                           {"V^T tiles", (const char*)vt, vt_bytes(BH, Nk, D), false},
                           {"K exponents", (const char*)kexp, tile_exp_bytes(BH, Nk), false},
                           {"V exponents", (const char*)vexp, tile_exp_bytes(BH, Nk), false},
                           {"range words", (const char*)flags, words_of_range(BH, work), true},
                           {"out", (const char*)out, (size_t)BH * q_rows * D * 2, true}};
  return check(r, "launch_dense_attn");
}

int launch_window_attn(const WindowAttnArgs& w, const int32_t* plan, const int32_t* wsum, const int32_t* bridge_idx,
                       const void* q, const void* k, const void* v, const void* rope, void* out, const WindowWs& ws,
                       stream_t) {
  if (w.ny < 1 || w.nx < 1 || w.ny > kMaxAxisWindows || w.nx > kMaxAxisWindows || w.max_windows != 4 * w.ny * w.nx)
    return fail(AREA_E_HIP, "launch_window_attn: window counts inconsistent");
  const int R = bridge_idx ? w.R : 0;
  const size_t seq = (size_t)w.BH * ((size_t)w.T + (size_t)w.Gh * w.Gw) * w.D * 2;
  const size_t q_total = (size_t)w.ny * w.nx * w.Ly * w.Lx;
  std::vector<Region> r = {
      {"plan", (const char*)plan, (AREA_PLAN_HEADER + (size_t)AREA_PLAN_REC * w.max_windows) * 4, false},
      {"wsum", (const char*)wsum, (size_t)w.Gh * w.Gw * 4, false},
      {"bridge_idx", (const char*)bridge_idx, (size_t)w.BH * R * 4, false},
      {"q", (const char*)q, seq, false},
      {"k", (const char*)k, seq, false},
      {"v", (const char*)v, seq, false},
      {"rope table", (const char*)rope, rope_table_bytes(w.Gh, w.Gw, w.D), false},
      {"out", (const char*)out, seq, true},
      {"items", (const char*)ws.items, window_items_ws_bytes(w.max_windows, w.max_items, w.ny * w.nx, w.max_gtiles),
       true},
      {"blend slots", (const char*)ws.slots, q_total * w.BH * w.D * 4, true},
      {"gathered keys", (const char*)ws.kg, (size_t)w.BH * w.max_gtiles * kAttnBN * w.D * 2, true},
      {"gathered V^T", (const char*)ws.vg, (size_t)w.BH * w.max_gtiles * kAttnBN * w.D * 2, true},
      {"bridge lists", (const char*)ws.blist, (size_t)w.max_windows * w.BH * R * 4, true},
      {"bridge counts", (const char*)ws.bcount, (size_t)w.max_windows * w.BH * 4, true},
      {"K exponents", (const char*)ws.kexp, (size_t)w.BH * w.max_gtiles * 4, true},
      {"V exponents", (const char*)ws.vexp, (size_t)w.BH * w.max_gtiles * 4, true},
      {"range words", (const char*)ws.flags, words_of_range(w.BH, w.BH * w.max_items), true}};
  return check(r, "launch_window_attn");
}

int measure_mfma_peak(void* sink, double* tflops, void*) {
  std::vector<Region> r = {{"sink", (const char*)sink, 4, false}};
  *tflops = 0.0;
  return check(r, "measure_mfma_peak");
}

}  // namespace area

// Host stand-in of the static-scratch plan call (the library's device array
// lives in a HIP source this build leaves out): the same validation and
// size limit, with a host array in place of the device one.
extern "C" int area_window_plan_static(const area_problem* p, int step, const int32_t* energy_q, const void* k,
                                       int32_t* plan, int32_t* wsum, int32_t* bridge_idx, void* stream) {
  constexpr size_t kScratchBytes = (size_t)16 << 20;
  alignas(256) static unsigned char scratch[kScratchBytes];
  int rc = area_validate(p);
  if (rc) return rc;
  if (area_workspace_bytes(p, AREA_OP_PLAN) > kScratchBytes)
    return area::fail(AREA_E_WORKSPACE, "the plan needs more than the static scratch");
  return area_window_plan(p, step, energy_q, k, plan, wsum, bridge_idx, scratch, kScratchBytes, stream);
}
