// Phase II window plan and global-KV bridge selection on gfx950.
//
// Every decision here is integer or fixed-order float64 so that the plan,
// the blend-weight sums and the bridge indices are reproducible bit for bit
// by any implementation of the same steps.
#include <hip/hip_runtime.h>

#include <string>

#include "area_internal.h"

namespace area {

namespace {

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(AREA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return AREA_OK;
}

// Workspace of the plan: int64 score per base window + the grid total,
// then one split flag per base window.
struct PlanWs {
  long long* scores;  // [n_base + 1]
  int* split;         // [n_base]
};

PlanWs plan_ws(void* ws, int n_base) {
  PlanWs p;
  p.scores = (long long*)ws;
  p.split = (int*)((char*)ws + align_up(sizeof(long long) * (n_base + 1)));
  return p;
}

template <typename T>
__device__ T block_sum(T v, T* red) {
  int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) red[wid] = v;
  __syncthreads();
  T s = 0;
  if (threadIdx.x == 0) {
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
    red[0] = s;
  }
  __syncthreads();
  s = red[0];
  __syncthreads();
  return s;
}

// Block b < n_base: S_w = sum over the base window's tokens (y, x) of
// E_q[y/2][x/2].  Block n_base: S_tot = the same sum over the whole grid
// (4 x the cell sum, every cell covering 2x2 tokens).
__global__ __launch_bounds__(256) void plan_scores_kernel(PlanArgs a, const int32_t* __restrict__ eq,
                                                          long long* __restrict__ scores) {
  __shared__ long long red[4];
  int nb = a.ny * a.nx;
  int b = blockIdx.x;
  int hw = a.Gw / 2;
  long long acc = 0;
  if (b < nb) {
    int y0 = a.ys[b / a.nx], x0 = a.xs[b % a.nx];
    int64_t area = (int64_t)a.Ly * a.Lx;
    for (int64_t i = threadIdx.x; i < area; i += blockDim.x) {
      int y = y0 + (int)(i / a.Lx), x = x0 + (int)(i % a.Lx);
      acc += eq[(int64_t)(y >> 1) * hw + (x >> 1)];
    }
  } else {
    int64_t cells = (int64_t)(a.Gh / 2) * hw;
    for (int64_t i = threadIdx.x; i < cells; i += blockDim.x) acc += eq[i];
    acc *= 4;
  }
  acc = block_sum<long long>(acc, red);
  if (threadIdx.x == 0) scores[b] = acc;
}

// Split test: den * S_w * N < num * S_tot * |Q_w| in 128-bit integers.
__device__ inline bool split_test(long long Sw, long long Stot, long long N, long long area, int num, int den) {
  unsigned __int128 lhs = (unsigned __int128)(unsigned long long)den * (unsigned long long)Sw;
  lhs *= (unsigned long long)N;
  unsigned __int128 rhs = (unsigned __int128)(unsigned long long)num * (unsigned long long)Stot;
  rhs *= (unsigned long long)area;
  return lhs < rhs;
}

// SplitMix64 (Steele, Lea, Flood 2014): k-th output from state `seed`.
__device__ inline unsigned long long splitmix64_dev(unsigned long long seed, unsigned long long k) {
  unsigned long long z = seed + k * 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

// Halo width of one window: fixed, or (READING R18: the seed controls the
// Halo widths, up to delta_max) drawn from 1..halo_max on a stream of its
// own, keyed by step, base window and quadrant (-1 when unsplit).
__device__ inline int halo_of(const PlanArgs& a, int base, int quadrant) {
  if (a.halo_max <= 0) return a.halo;
  const unsigned long long key = 1ULL + ((unsigned long long)a.t * 4096ULL + (unsigned long long)base) * 5ULL +
                                 (unsigned long long)(quadrant + 1);
  return 1 + (int)(splitmix64_dev(a.seed ^ 0x48414C4FULL, key) % (unsigned long long)a.halo_max);
}

// One block: split decisions, canonical record order, Halo rectangles and
// the plan header.
__global__ __launch_bounds__(256) void plan_emit_kernel(PlanArgs a, const long long* __restrict__ scores,
                                                        int* __restrict__ split, int32_t* __restrict__ plan) {
  __shared__ int s_first[kMaxAxisWindows * kMaxAxisWindows];
  __shared__ int s_nwin, s_nsplit;
  int nb = a.ny * a.nx;
  long long N = (long long)a.Gh * a.Gw;
  long long area = (long long)a.Ly * a.Lx;
  bool can_split = a.split_den > 0 && a.Ly >= 2 && a.Lx >= 2;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    int sp = 0;
    if (can_split) sp = split_test(scores[b], scores[nb], N, area, a.split_num, a.split_den) ? 1 : 0;
    split[b] = sp;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int r = 0, ns = 0;
    for (int b = 0; b < nb; ++b) {
      s_first[b] = r;
      r += split[b] ? 4 : 1;
      ns += split[b];
    }
    s_nwin = r;
    s_nsplit = ns;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    int y0 = a.ys[b / a.nx], x0 = a.xs[b % a.nx];
    int rects[4][5];
    int nr;
    if (split[b]) {
      int h1 = a.Ly / 2, w1 = a.Lx / 2;
      int r0[4][5] = {{y0, x0, h1, w1, 0},
                      {y0, x0 + w1, h1, a.Lx - w1, 1},
                      {y0 + h1, x0, a.Ly - h1, w1, 2},
                      {y0 + h1, x0 + w1, a.Ly - h1, a.Lx - w1, 3}};
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 5; ++j) rects[i][j] = r0[i][j];
      nr = 4;
    } else {
      rects[0][0] = y0; rects[0][1] = x0; rects[0][2] = a.Ly; rects[0][3] = a.Lx; rects[0][4] = -1;
      nr = 1;
    }
    for (int i = 0; i < nr; ++i) {
      int ry = rects[i][0], rx = rects[i][1], rh = rects[i][2], rw = rects[i][3];
      const int d = halo_of(a, b, rects[i][4]);
      int ky0 = max(0, ry - d), kx0 = max(0, rx - d);
      int ky1 = min(a.Gh, ry + rh + d), kx1 = min(a.Gw, rx + rw + d);
      int32_t* rec = plan + AREA_PLAN_HEADER + (int64_t)AREA_PLAN_REC * (s_first[b] + i);
      rec[0] = ry; rec[1] = rx; rec[2] = rh; rec[3] = rw;
      rec[4] = ky0; rec[5] = kx0; rec[6] = ky1 - ky0; rec[7] = kx1 - kx0;
      rec[8] = b; rec[9] = rects[i][4];
    }
  }
  if (threadIdx.x == 0) {
    int32_t* h = plan;
    for (int i = 0; i < AREA_PLAN_HEADER; ++i) h[i] = 0;
    h[AREA_PH_NWIN] = s_nwin;
    h[AREA_PH_STEP] = a.t;
    h[AREA_PH_W] = a.w;
    h[AREA_PH_NY] = a.ny;
    h[AREA_PH_NX] = a.nx;
    h[AREA_PH_JITY] = a.jit_y;
    h[AREA_PH_JITX] = a.jit_x;
    h[AREA_PH_HALO] = a.halo;
    h[AREA_PH_R] = a.R;
    h[AREA_PH_NSPLIT] = s_nsplit;
    h[AREA_PH_QTOT] = (int32_t)((long long)nb * area);
  }
}

__device__ inline int tent_w(int u, int L) { return min(u + 1, L - u); }

// wsum[y*Gw + x] = sum over the windows covering (y, x) of the tent weight
// along y times along x (the quadrant of a split window when split).
__global__ __launch_bounds__(256) void plan_wsum_kernel(PlanArgs a, const int* __restrict__ split,
                                                        int32_t* __restrict__ wsum) {
  int64_t N = (int64_t)a.Gh * a.Gw;
  int h1 = a.Ly / 2, w1 = a.Lx / 2;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < N; p += (int64_t)gridDim.x * blockDim.x) {
    int y = (int)(p / a.Gw), x = (int)(p % a.Gw);
    int acc = 0;
    for (int i = 0; i < a.ny; ++i) {
      int uy = y - a.ys[i];
      if (uy < 0 || uy >= a.Ly) continue;
      for (int j = 0; j < a.nx; ++j) {
        int ux = x - a.xs[j];
        if (ux < 0 || ux >= a.Lx) continue;
        int wy, wx;
        if (split[i * a.nx + j]) {
          wy = uy < h1 ? tent_w(uy, h1) : tent_w(uy - h1, a.Ly - h1);
          wx = ux < w1 ? tent_w(ux, w1) : tent_w(ux - w1, a.Lx - w1);
        } else {
          wy = tent_w(uy, a.Ly);
          wx = tent_w(ux, a.Lx);
        }
        acc += wy * wx;
      }
    }
    wsum[p] = acc;
  }
}

// ---------------------------------------------------------------- bridge --
// Workspace: partial fixed-point key sums [BH][chunks][D] int64, the mean
// key [BH][D] float64, per-cell winners [BH][R] int32.
struct BridgeWs {
  long long* part;
  double* mean;
  int* cell;
};

// Keys saturate at this magnitude inside the mean-key sum only.
constexpr float kMeanClamp = 268435456.0f;  // 2^28, exact in fp32

BridgeWs bridge_ws(void* ws, int64_t BH, int N, int D, int R) {
  BridgeWs b;
  char* p = (char*)ws;
  b.part = (long long*)p;
  p += align_up(sizeof(long long) * BH * bridge_chunks(N) * D);
  b.mean = (double*)p;
  p += align_up(sizeof(double) * BH * D);
  b.cell = (int*)p;
  return b;
}

// Fixed-point sums round_half_even(k * 2^24) over one chunk of rows for
// every channel, keys saturated at +-2^28 (|term| <= 2^52, so a chunk of
// 1024 rows sums exactly in int64).  Thread t reads 8 channels (16 bytes) of
// a row; 16 consecutive threads cover one 128-channel row.
template <int D>
__global__ __launch_bounds__(256) void bridge_sum_kernel(const uint4* __restrict__ k, long long* __restrict__ part,
                                                         int N, int T) {
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;         // rows per pass
  __shared__ long long red[RPP][D];
  int chunk = blockIdx.x;
  int64_t bh = blockIdx.y;
  int c = threadIdx.x % CPR, rr = threadIdx.x / CPR;
  long long acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int r0 = chunk * kBridgeChunk, r1 = min(N, r0 + kBridgeChunk);
  const uint4* base = k + (bh * (int64_t)(T + N) + T) * CPR;  // the image rows of the sequence
  // four rows in flight per thread; rows past the chunk read as zero keys
  for (int r = r0 + rr; r < r1; r += 4 * RPP) {
    uint4 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rj = r + j * RPP;
      w[j] = rj < r1 ? base[(int64_t)rj * CPR + c] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned u[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double lo = (double)fminf(fmaxf(__uint_as_float(u[i] << 16), -kMeanClamp), kMeanClamp);
        const double hi = (double)fminf(fmaxf(__uint_as_float(u[i] & 0xFFFF0000u), -kMeanClamp), kMeanClamp);
        acc[2 * i] += (long long)rint(lo * 16777216.0);
        acc[2 * i + 1] += (long long)rint(hi * 16777216.0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rr][8 * c + i] = acc[i];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    long long s = 0;
    for (int i = 0; i < RPP; ++i) s += red[i][d];
    part[((int64_t)bh * gridDim.x + chunk) * D + d] = s;
  }
}

// mean_d = T / (2^24 N): T, the sum of the fixed-point keys, exact in 128
// bits, rounded once to float64 as hi * 2^32 + lo (hi = floor(T / 2^32) and
// lo = T mod 2^32 are exact doubles), then one float64 division.
__global__ void bridge_mean_kernel(const long long* __restrict__ part, double* __restrict__ mean, int nch, int N,
                                   int D) {
  int64_t bh = blockIdx.x;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    // eight independent partial sums keep eight chunk loads in flight
    const long long* pd = part + (int64_t)bh * nch * D + d;
    __int128 p[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int c = 0;
    for (; c + 8 <= nch; c += 8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] += pd[(int64_t)(c + j) * D];
    }
    for (; c < nch; ++c) p[0] += pd[(int64_t)c * D];
    __int128 s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += p[j];
    const long long hi = (long long)(s >> 32);
    const unsigned lo = (unsigned)(s & 0xFFFFFFFF);
    mean[bh * D + d] = ((double)hi * 4294967296.0 + (double)lo) / (16777216.0 * (double)N);
  }
}

// One block per (batch*head, cell): score every token of the cell by
// sum over channels (ascending) of (k - mean)^2 in float64 without
// contraction, keep the largest score, ties to the smaller token index.
template <int D>
__global__ __launch_bounds__(256) void bridge_cell_kernel(const unsigned short* __restrict__ k,
                                                          const double* __restrict__ mean, int* __restrict__ cell_out,
                                                          int Gh, int Gw, int rh, int rw, int T) {
#pragma clang fp contract(off)
  __shared__ double mu[D];
  __shared__ double best_s[4];
  __shared__ int best_i[4];
  int cell = blockIdx.x;
  int64_t bh = blockIdx.y;
  int R = rh * rw;
  for (int d = threadIdx.x; d < D; d += blockDim.x) mu[d] = mean[bh * D + d];
  __syncthreads();
  int a = cell / rw, c = cell % rw;
  int y0 = (int)((int64_t)a * Gh / rh), y1 = (int)((int64_t)(a + 1) * Gh / rh);
  int x0 = (int)((int64_t)c * Gw / rw), x1 = (int)((int64_t)(c + 1) * Gw / rw);
  int cw = x1 - x0;
  int ncell = (y1 - y0) * cw;
  const unsigned short* kb = k + (bh * ((int64_t)Gh * Gw + T) + T) * D;  // the image rows of the sequence
  double bs = -1.0;
  int bi = 0x7FFFFFFF;
  for (int i = threadIdx.x; i < ncell; i += blockDim.x) {
    int n = (y0 + i / cw) * Gw + x0 + i % cw;
    const uint4* row = reinterpret_cast<const uint4*>(kb + (int64_t)n * D);
    double s = 0.0;
#pragma unroll 4
    for (int q = 0; q < D / 8; ++q) {
      uint4 w = row[q];
      const unsigned u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        double t0 = (double)__uint_as_float(u[j] << 16) - mu[8 * q + 2 * j];
        double p0 = t0 * t0;
        s = s + p0;
        double t1 = (double)__uint_as_float(u[j] & 0xFFFF0000u) - mu[8 * q + 2 * j + 1];
        double p1 = t1 * t1;
        s = s + p1;
      }
    }
    if (s > bs || (s == bs && n < bi)) {
      bs = s;
      bi = n;
    }
  }
  // wave-level then block-level arg-max
  for (int o = 32; o > 0; o >>= 1) {
    double os = __shfl_xor(bs, o);
    int oi = __shfl_xor(bi, o);
    if (os > bs || (os == bs && oi < bi)) {
      bs = os;
      bi = oi;
    }
  }
  int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) {
    best_s[wid] = bs;
    best_i[wid] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) {
      if (best_s[w] > bs || (best_s[w] == bs && best_i[w] < bi)) {
        bs = best_s[w];
        bi = best_i[w];
      }
    }
    cell_out[bh * R + cell] = bi;
  }
}

// Ascending order of the R winners of one (batch*head).  Cell (a, c) sits at
// a * rw + c and cell row a covers grid rows [a Gh / rh, (a+1) Gh / rh), so
// every winner of a cell row precedes every winner of the next: sorting each
// row of rw cells in place (bitonic, in LDS) sorts the whole list.  One block
// per (cell row, batch*head).
__global__ __launch_bounds__(1024) void bridge_sort_kernel(const int* __restrict__ cell, int* __restrict__ idx,
                                                           int rh, int rw) {
  __shared__ int s[kBridgeSortMax];
  const int64_t row = blockIdx.x, bh = blockIdx.y;
  const int64_t base = bh * (int64_t)rh * rw + row * rw;
  int P = 1;
  while (P < rw) P <<= 1;
  for (int i = threadIdx.x; i < P; i += blockDim.x) s[i] = i < rw ? cell[base + i] : 0x7FFFFFFF;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += blockDim.x) {
        int l = i ^ j;
        if (l > i) {
          bool up = (i & k) == 0;
          int x = s[i], y = s[l];
          if ((x > y) == up) {
            s[i] = y;
            s[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < rw; i += blockDim.x) idx[base + i] = s[i];
}

}  // namespace

int launch_plan(const PlanArgs& a, const int32_t* energy_q, int32_t* plan, int32_t* wsum, void* ws,
                stream_t s) {
  hipStream_t st = (hipStream_t)s;
  int nb = a.ny * a.nx;
  PlanWs w = plan_ws(ws, nb);
  if (a.split_den > 0) {
    hipLaunchKernelGGL(plan_scores_kernel, dim3(nb + 1), dim3(256), 0, st, a, energy_q, w.scores);
    int rc = check_launch("plan_scores_kernel");
    if (rc) return rc;
  }
  hipLaunchKernelGGL(plan_emit_kernel, dim3(1), dim3(256), 0, st, a, (const long long*)w.scores, w.split, plan);
  int rc = check_launch("plan_emit_kernel");
  if (rc) return rc;
  int64_t N = (int64_t)a.Gh * a.Gw;
  int grid = (int)std::min<int64_t>((N + 255) / 256, 65536);
  hipLaunchKernelGGL(plan_wsum_kernel, dim3(grid), dim3(256), 0, st, a, (const int*)w.split, wsum);
  return check_launch("plan_wsum_kernel");
}

int launch_bridge(const void* k, int32_t* idx, int64_t BH, int T, int Gh, int Gw, int D, int R, int rh, int rw,
                  void* ws, stream_t s) {
  hipStream_t st = (hipStream_t)s;
  int N = Gh * Gw;
  BridgeWs b = bridge_ws(ws, BH, N, D, R);
  int nch = bridge_chunks(N);
  if (BH > 65535) return fail(AREA_E_UNSUPPORTED, "batch*heads above 65535");
  if (D == 128)
    hipLaunchKernelGGL(bridge_sum_kernel<128>, dim3(nch, (unsigned)BH), dim3(256), 0, st, (const uint4*)k, b.part, N,
                       T);
  else
    hipLaunchKernelGGL(bridge_sum_kernel<64>, dim3(nch, (unsigned)BH), dim3(256), 0, st, (const uint4*)k, b.part, N,
                       T);
  int rc = check_launch("bridge_sum_kernel");
  if (rc) return rc;
  hipLaunchKernelGGL(bridge_mean_kernel, dim3((unsigned)BH), dim3(128), 0, st, (const long long*)b.part, b.mean,
                     nch, N, D);
  rc = check_launch("bridge_mean_kernel");
  if (rc) return rc;
  if (D == 128)
    hipLaunchKernelGGL(bridge_cell_kernel<128>, dim3(R, (unsigned)BH), dim3(256), 0, st, (const unsigned short*)k,
                       (const double*)b.mean, b.cell, Gh, Gw, rh, rw, T);
  else
    hipLaunchKernelGGL(bridge_cell_kernel<64>, dim3(R, (unsigned)BH), dim3(256), 0, st, (const unsigned short*)k,
                       (const double*)b.mean, b.cell, Gh, Gw, rh, rw, T);
  rc = check_launch("bridge_cell_kernel");
  if (rc) return rc;
  if (rw > kBridgeSortMax || rh > 65535) return fail(AREA_E_UNSUPPORTED, "bridge cell grid too large");
  hipLaunchKernelGGL(bridge_sort_kernel, dim3((unsigned)rh, (unsigned)BH), dim3(1024), 0, st, (const int*)b.cell,
                     idx, rh, rw);
  return check_launch("bridge_sort_kernel");
}

}  // namespace area
