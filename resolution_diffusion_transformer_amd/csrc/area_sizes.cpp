// Sizes of the kernels' workspace regions: host arithmetic only, kept apart
// from the kernel sources so that the host-only (sanitizer) build of the
// library sizes every region exactly as the library does.
#include <algorithm>

#include "area_internal.h"

namespace area {

// (cos, sin) tables: [P][D/4] float2 then [D/8][P] float4, P = max(Gh, Gw).
size_t rope_table_bytes(int Gh, int Gw, int D) { return 2 * (size_t)std::max(Gh, Gw) * (D / 4) * 2 * sizeof(float); }

// fp16 V^T tiles of 64 keys, zero padded.
size_t vt_bytes(int64_t BH, int M, int D) { return (size_t)BH * ((M + kAttnBN - 1) / kAttnBN) * kAttnBN * D * 2; }

// One int32 exponent per (batch*head, 64-key tile).
size_t tile_exp_bytes(int64_t BH, int M) { return (size_t)BH * ((M + kAttnBN - 1) / kAttnBN) * sizeof(int); }

// Window work structures: item and gather-tile counters, per-record slot and
// key-tile offsets, the first record of each base window, the (record, query
// tile) and (record, key tile) lists.
size_t window_items_ws_bytes(int max_windows, int64_t max_items, int n_base, int64_t max_gtiles) {
  return align_up(2 * sizeof(int)) + 2 * align_up(sizeof(int) * (max_windows > 0 ? max_windows : 1)) +
         align_up(sizeof(int) * (n_base > 0 ? n_base : 1)) + align_up(sizeof(int) * 2 * (max_items > 0 ? max_items : 1)) +
         align_up(sizeof(int) * 2 * (max_gtiles > 0 ? max_gtiles : 1));
}

// Plan: an int64 score per base window plus the grid total, a split flag
// per base window.
size_t plan_ws_bytes(int n_base) {
  return align_up(sizeof(long long) * (n_base + 1)) + align_up(sizeof(int) * (n_base > 0 ? n_base : 1));
}

int bridge_chunks(int N) { return (N + kBridgeChunk - 1) / kBridgeChunk; }

// Bridge: int64 partial key sums per chunk, the float64 mean key, one winner
// per cell.
size_t bridge_ws_bytes(int64_t BH, int N, int D, int R) {
  if (R <= 0) return 0;
  return align_up(sizeof(long long) * BH * bridge_chunks(N) * D) + align_up(sizeof(double) * BH * D) +
         align_up(sizeof(int) * BH * R);
}

}  // namespace area
