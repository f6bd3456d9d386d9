// Internal declarations shared by the host code and the kernel launchers of
// the AReA library.  Nothing here is part of the public ABI (include/area.h).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "area.h"

namespace area {

// ---------------------------------------------------------------- errors --
void set_error(const std::string& msg);
int fail(int status, const std::string& msg);

// ------------------------------------------------------- fixed constants --
constexpr int kMaxAxisWindows = 64;    // base windows per axis (kernel-argument table)
constexpr int kMaxGridSide = 65536;    // tokens per grid side (RoPE table rows)
constexpr int kAttnQG = 1;             // 32-query groups per attention wave
constexpr int kAttnWaves = 8;          // waves per attention work-group
constexpr int kAttnBM = 32 * kAttnQG * kAttnWaves;  // queries per attention work item
constexpr int kAttnBN = 64;            // keys per staged tile
constexpr int kBridgeChunk = 1024;     // rows per partial mean-key sum
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// --------------------------------------------------------- schedule math --
// All plan decisions are integer or fixed-order float64 so that any other
// implementation of the same steps reproduces them exactly.

int gcd_int(int a, int b);
// Common divisor d >= lo of (a, b) nearest to num/den, ties to the larger;
// -1 if none.
int nearest_common_divisor(int a, int b, int lo, long long num, long long den);
int derive_f0(const area_problem& p);              // READING R5
int ramp_factor(const area_problem& p, int f0, int t);  // READING R4
int w_start_of(const area_problem& p);            // READING R7
int window_side(const area_problem& p, int t);     // READING R6
int bridge_size(const area_problem& p, int w);     // READING R19
void base_starts(int G, int w, std::vector<int>& out);  // READING R8
uint64_t splitmix64(uint64_t seed, uint64_t k);
int jitter_offset(const std::vector<int>& starts, int L, uint64_t seed, int t, int axis);  // R9

struct AxisTiling {
  int n = 0;
  int L = 0;          // window extent along the axis (min(w, G))
  int jitter = 0;
  int start[kMaxAxisWindows];
};
// Base tiling + shift of one axis for Phase II step t; false if more than
// kMaxAxisWindows windows would be needed.
bool axis_tiling(int G, int w, uint64_t seed, int t, int axis, AxisTiling& out);

bool bridge_cells(int R, int Gh, int Gw, int& rh, int& rw);  // READING R13

bool canvas_gated(const area_problem& p);  // at or below native: full attention

// Base-window statistics of a Phase II step used to size launches.
struct WindowStepInfo {
  int t = 0;                 // Phase II step index
  int w = 0;
  AxisTiling ty, tx;
  int64_t q_total = 0;       // sum of query areas (== with splits)
  int64_t max_items = 0;     // work items (window, query tile) over all split choices
  int64_t max_gtiles = 0;    // gathered 64-key tiles over all split choices
  int R = 0;                 // bridge tokens per (batch, head) of the step
};
int window_step(const area_problem& p, int step, WindowStepInfo& out);

// Events recorded around attention-kernel launches (area_set_attn_events).
struct AttnEvents {
  void* begin = nullptr;
  void* end = nullptr;
};
AttnEvents& attn_events();

// Register-only MFMA stream timed on `stream` (area_measure_mfma_peak).
int measure_mfma_peak(void* sink, double* tflops, void* stream);

// ---------------------------------------------------------- launchers ----
// Each returns AREA_OK or AREA_E_HIP (with the error text set).  Arguments
// have been validated by the caller.
typedef void* stream_t;

// (cos, sin) tables of every axis position p < P = max(Gh, Gw) and
// frequency k < D/4 at angle (p / div) * theta^(-4k/D), fp32: first
// [P][D/4] float2 (the key conversions turn keys through it), then
// [D/8][P] float4 of frequency pairs (the attention kernels turn queries
// through it).  The same launch clears the n_flags words at `flags` (the
// per-(batch, head) range flags of the call's key and value tiles).
size_t rope_table_bytes(int Gh, int Gw, int D);
int launch_rope_table(void* tab, int Gh, int Gw, int D, float theta, float div, int* flags, int64_t n_flags,
                      stream_t s);
int launch_pool(const void* k, const void* v, void* kp, void* vp, int64_t BH, int T, int Gh, int Gw,
                int D, int f, int mode, unsigned long long seed, float theta, stream_t s);
int launch_dwt(const float* latent, float* energy, int32_t* energy_q, int C, int Gh, int Gw,
               stream_t s);

struct PlanArgs {
  int Gh, Gw, halo, R, split_num, split_den, t, w;
  int halo_max;                  // > 0: per-window Halo widths drawn from 1..halo_max
  unsigned long long seed;
  int ny, nx, jit_y, jit_x, Ly, Lx;
  int ys[kMaxAxisWindows];
  int xs[kMaxAxisWindows];
};
int launch_plan(const PlanArgs& a, const int32_t* energy_q, int32_t* plan, int32_t* wsum,
                void* ws, stream_t s);
size_t plan_ws_bytes(int n_base);

int launch_bridge(const void* k, int32_t* idx, int64_t BH, int T, int Gh, int Gw, int D, int R, int rh,
                  int rw, void* ws, stream_t s);
constexpr int kBridgeSortMax = 4096;  // cells per row of the bridge cell grid
size_t bridge_ws_bytes(int64_t BH, int N, int D, int R);
int bridge_chunks(int N);             // kBridgeChunk-row partial sums of the mean key

// Dense key/value operands, one 64-key tile per work-group: fp16 key rows
// kr[bh][M][D] and fp16 V^T tiles vt[bh][t][d][k] = v[bh][64 t + k][d]
// (zero padded), each tile scaled by its own power of two 2^-e with e in
// kexp / vexp[bh][t] (0 for magnitudes in [2^-8, 2^15)); flags[bh] is set
// when a tile of (b, h) has a nonzero exponent.  k and v are [BH][M][D]:
// bf16 sequences (T text rows, then the Gh x Gw grid; keys turned by RoPE
// through the first table of launch_rope_table) or, with f32_in, fp32 pooled
// rows whose keys are already turned.
size_t vt_bytes(int64_t BH, int M, int D);
size_t tile_exp_bytes(int64_t BH, int M);  // one int32 per (batch*head, 64-key tile)
int launch_kv_tiles(const void* k, const void* v, const void* rope, void* kr, void* vt, int* kexp, int* vexp,
                    int* flags, int64_t BH, int M, int D, bool f32_in, int T, int Gw, stream_t s);

// Attention of bf16 queries (turned by RoPE through the tables `rope` of
// launch_rope_table as they are loaded; rows below q_text are text, row
// q_text + n is image token n of the Gh x Gw grid) over the key rows and
// V^T tiles of launch_kv_tiles, bf16 output.  Queries are rows q0 .. q0 +
// Nq - 1 of sequences of q_rows rows (q and out share that layout); keys are
// the Nk rows of k_rot / vt per (batch, head).
int launch_dense_attn(const void* q, const void* rope, int q_text, int Gh, int Gw, const void* k_rot,
                      const void* vt, const int* kexp, const int* vexp, int* flags, void* out, int64_t BH,
                      int Nq, int q0, int q_rows, int Nk, int D, stream_t s);
// Words of the range region of an attention call: BH flags, the 8 per-XCD
// work counters of the persistent attention kernel, then the count and list
// of work items the scaled attention kernel runs.  The call's rope-table
// launch clears the first range_clear_words (flags, counters and count).
inline size_t range_words(int64_t BH, int64_t work) { return (size_t)BH + 8 + 1 + (size_t)work; }
inline int64_t range_clear_words(int64_t BH) { return BH + 8 + 1; }

struct WindowAttnArgs {
  int Gh, Gw, D, R;
  int T;                          // text tokens ahead of the image rows, joined to every key set
  int64_t BH;
  int max_windows;
  int64_t max_items, max_gtiles;
  int ny, nx;
  int ys[kMaxAxisWindows], xs[kMaxAxisWindows];
  int Ly, Lx;
};
// Workspace regions of the windowed attention.
struct WindowWs {
  void* items;     // window_items_ws_bytes
  float* slots;    // [q_total][BH][D] fp32
  void* kg;        // [BH][max_gtiles * 64][D] fp16 gathered keys
  void* vg;        // [BH][max_gtiles][D][64] fp16 gathered V^T tiles
  int* blist;      // [max_windows][BH][R] kept bridge tokens
  int* bcount;     // [max_windows][BH]
  int* kexp;       // [BH][max_gtiles] power-of-two exponent of each gathered key tile
  int* vexp;       // [BH][max_gtiles] the same for the V^T tiles
  int* flags;      // range_words(BH, BH * max_items): flags set by the gather, then the scaled items
};
// q, k, v: un-rotated bf16 sequences; the gather turns the keys and the
// attention kernel the queries by RoPE through the tables `rope` of
// launch_rope_table (div 1).
int launch_window_attn(const WindowAttnArgs& a, const int32_t* plan, const int32_t* wsum,
                       const int32_t* bridge_idx, const void* q, const void* k, const void* v,
                       const void* rope, void* out, const WindowWs& ws, stream_t s);
size_t window_items_ws_bytes(int max_windows, int64_t max_items, int n_base, int64_t max_gtiles);

}  // namespace area
