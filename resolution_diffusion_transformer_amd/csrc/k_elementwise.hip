// Bandwidth-bound kernels of the AReA path on gfx950: the two-axis RoPE
// (cos, sin) tables and the fp16 rotation of dense keys, f x f key/value
// pooling with RoPE at coarse positions, and the Haar detail-energy map.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <string>

#include "area_internal.h"

namespace area {

namespace {

struct InvFreq {
  float v[32];  // theta^(-4k/D), k < D/4 (D <= 128)
};

InvFreq make_inv_freq(int D, float theta) {
  InvFreq f;
  int half = D / 2;
  for (int k = 0; k < 32; ++k) {
    f.v[k] = k < half / 2 ? (float)std::pow((double)theta, -2.0 * k / (double)half) : 0.0f;
  }
  return f;
}

// 8 bf16 channels (16 bytes) to fp32 (exact).
__device__ inline void unpack8(const uint4& r, float* x) {
  const unsigned w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// 8 channels as fp32 into the two float4 of chunk i of a row-major fp32 buffer.
__device__ inline void store8_f32(float4* dst, int64_t i, const float* x) {
  dst[2 * i] = make_float4(x[0], x[1], x[2], x[3]);
  dst[2 * i + 1] = make_float4(x[4], x[5], x[6], x[7]);
}

// k-th output of the SplitMix64 generator (Steele, Lea and Flood, OOPSLA
// 2014) started from `seed`: golden-gamma increment, variant-13 finalizer.
__device__ inline unsigned long long splitmix64(unsigned long long seed, unsigned long long k) {
  unsigned long long z = seed + k * 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

// Random pooling (READING R21): one in-block offset per (pooling factor,
// block), drawn on its own SplitMix64 stream ("POOL"), shared by every
// batch, head, K and V.
constexpr unsigned long long kPoolStream = 0x504F4F4CULL;

__device__ inline int random_pool_offset(unsigned long long seed, int f, long long block) {
  const unsigned long long key = 1ULL + ((unsigned long long)f << 32) + (unsigned long long)block;
  return (int)(splitmix64(seed ^ kPoolStream, key) % (unsigned long long)(f * f));
}

// Rotation of the 8 channels [8c, 8c+8) of a token at grid position
// (py, px): channels below D/2 follow the row, the others the column; pair
// (2k, 2k+1) of an axis half turns by pos * inv_freq[k].  rope_cs computes
// the four (cos, sin) pairs once, rope_apply turns one vector by them.
struct Rot4 {
  float co[4], sn[4];
};

__device__ inline Rot4 rope_cs(int c, int D, float py, float px, const InvFreq& f) {
  Rot4 r;
  int d0 = 8 * c;
  int half = D / 2;
  float pos = d0 < half ? py : px;
  int k0 = (d0 % half) / 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) sincosf(pos * f.v[k0 + j], &r.sn[j], &r.co[j]);
  return r;
}

__device__ inline void rope_apply(float* x, const Rot4& r) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = x[2 * j], b = x[2 * j + 1];
    x[2 * j] = a * r.co[j] - b * r.sn[j];
    x[2 * j + 1] = a * r.sn[j] + b * r.co[j];
  }
}

// (cos, sin) of every (axis position, frequency) pair the attention kernels
// rotate by, c_k(p) = sincos((p / div) * inv_freq[k]) for p < P, k < D/4, in
// two layouts: tab[p][k] (float2; a thread's chunk of one token reads
// neighbouring frequencies, the windowed gather's access) and
// tabq[k / 2][p] (float4 = c_k, c_k+1 for even k; lanes holding neighbouring
// positions read neighbouring entries, the attention kernels' query load).
// Angles are formed as rope_cs forms those of the pooled keys: the fp32
// position times the fp32 inverse frequency, then sincosf.
// The same launch clears the call's n_flags range-flag words (grid-strided).
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ tab, float2* __restrict__ tabq, int P,
                                                         int NF, float div, InvFreq f, int* __restrict__ flags,
                                                         int64_t n_flags) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = e; i < n_flags; i += (int64_t)gridDim.x * blockDim.x) flags[i] = 0;
  if (e >= P * NF) return;
  const int p = e / NF, k = e - p * NF;
  const float pos = (float)p / div;
  float sn, co;
  sincosf(pos * f.v[k], &sn, &co);
  tab[e] = make_float2(co, sn);
  tabq[((k >> 1) * P + p) * 2 + (k & 1)] = make_float2(co, sn);
}

// The first T output rows are the text keys and values, copied unpooled and
// unrotated (text sits at position (0, 0)).  For a pooled row, mean mode
// sums the block's f*f tokens in fp32 (block rows in order, then columns)
// and divides by f*f; centre mode takes token (f/2, f/2) of the block and
// random mode the token at its seeded offset (medoid mode has a kernel of its
// own below).  Keys are then rotated at the coarse position (by, bx); values
// are not rotated.
// The pooled rows are written in fp32 (the f*f sum and the division in fp32,
// no further rounding).
// Grid: x over the (output row, chunk) pairs of one (batch, head), y over
// (batch, head), both grid-strided.
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                   float4* __restrict__ kp, float4* __restrict__ vp, int64_t BH,
                                                   int Gh, int Gw, int f, int mode, int T, unsigned long long seed,
                                                   InvFreq fr) {
  constexpr int CPT = D / 8;
  const int Wp = Gw / f, Hp = Gh / f;
  const int64_t per_bh = ((int64_t)T + (int64_t)Hp * Wp) * CPT;  // output chunks per (batch, head)
  const int64_t L = T + (int64_t)Gh * Gw;                          // input rows per (batch, head)
  for (int64_t bh = blockIdx.y; bh < BH; bh += gridDim.y) {
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < per_bh;
         j += (int64_t)gridDim.x * blockDim.x) {
      const int c = (int)(j & (CPT - 1));
      const int64_t r = j / CPT;
      const int64_t i = bh * per_bh + j;
      float ks[8], vs[8];
      if (r < T) {
        unpack8(k[(bh * L + r) * CPT + c], ks);
        unpack8(v[(bh * L + r) * CPT + c], vs);
        store8_f32(kp, i, ks);
        store8_f32(vp, i, vs);
        continue;
      }
      const int np = (int)(r - T);
      const int by = np / Wp, bx = np - (np / Wp) * Wp;
      const uint4* kb = k + (bh * L + T) * CPT + c;
      const uint4* vb = v + (bh * L + T) * CPT + c;
      if (mode == AREA_POOL_CENTER || mode == AREA_POOL_RANDOM) {
        const int o = mode == AREA_POOL_CENTER ? (f / 2) * f + f / 2 : random_pool_offset(seed, f, np);
        int64_t n = (int64_t)(by * f + o / f) * Gw + (bx * f + o % f);
        unpack8(kb[n * CPT], ks);
        unpack8(vb[n * CPT], vs);
      } else {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) ks[jj] = vs[jj] = 0.0f;
        for (int dy = 0; dy < f; ++dy) {
          int64_t row = (int64_t)(by * f + dy) * Gw + bx * f;
          for (int dx = 0; dx < f; ++dx) {
            float a[8], b[8];
            unpack8(kb[(row + dx) * CPT], a);
            unpack8(vb[(row + dx) * CPT], b);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              ks[jj] += a[jj];
              vs[jj] += b[jj];
            }
          }
        }
        float inv = (float)(f * f);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          ks[jj] = ks[jj] / inv;
          vs[jj] = vs[jj] / inv;
        }
      }
      rope_apply(ks, rope_cs(c, D, (float)by, (float)bx, fr));
      store8_f32(kp, i, ks);
      store8_f32(vp, i, vs);
    }
  }
}

// Medoid pooling (READING R22), one wave per output row of one (batch,
// head): rows below T copy the text token; pooled row T + b finds the medoid
// of block b -- the token whose un-rotated key has the smallest sum of
// Euclidean distances to the block's keys -- in float64 with every operation
// in the written order (no contraction): per pair, the squared differences
// summed over d ascending, the square root, then the sum over the other
// token ascending; ties go to the smaller row-major offset.  Lanes take the
// candidates in turn and a wave reduction picks the winner; then the row is
// written like the other modes: K rotated at the coarse position (by, bx),
// V unrotated, both fp32.
template <int D>
__global__ __launch_bounds__(64) void pool_medoid_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                         float4* __restrict__ kp, float4* __restrict__ vp, int64_t BH,
                                                         int Gh, int Gw, int f, int T, InvFreq fr) {
#pragma clang fp contract(off)
  constexpr int CPT = D / 8;
  const int lane = threadIdx.x;
  const int Wp = Gw / f;
  const int64_t rows_out = (int64_t)T + (int64_t)(Gh / f) * Wp;
  const int64_t L = T + (int64_t)Gh * Gw;
  const int64_t r = blockIdx.x;
  for (int64_t bh = blockIdx.y; bh < BH; bh += gridDim.y) {
    const uint4* kb = k + bh * L * CPT;
    const uint4* vb = v + bh * L * CPT;
    int64_t src;
    int by = 0, bx = 0;
    if (r < T) {
      src = r;
    } else {
      const int b = (int)(r - T);
      by = b / Wp;
      bx = b - by * Wp;
      const int n = f * f;
      auto tok = [&](int o) -> int64_t { return T + (int64_t)(by * f + o / f) * Gw + (bx * f + o % f); };
      double best = 0.0;
      int best_j = n;  // none yet
      for (int j = lane; j < n; j += 64) {
        const uint4* kj = kb + tok(j) * CPT;
        double total = 0.0;
        for (int i = 0; i < n; ++i) {
          const uint4* ki = kb + tok(i) * CPT;
          double s = 0.0;
          for (int c = 0; c < CPT; ++c) {
            float a[8], bv[8];
            unpack8(ki[c], a);
            unpack8(kj[c], bv);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const double diff = (double)a[e] - (double)bv[e];
              s = s + diff * diff;
            }
          }
          total = total + __builtin_sqrt(s);
        }
        if (best_j == n || total < best) {
          best = total;
          best_j = j;
        }
      }
      // wave argmin: the smaller total wins, equal totals go to the smaller offset
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const double ob = __shfl_xor(best, m);
        const int oj = __shfl_xor(best_j, m);
        const bool take = oj < n && (best_j == n || ob < best || (ob == best && oj < best_j));
        best = take ? ob : best;
        best_j = take ? oj : best_j;
      }
      src = tok(best_j);
    }
    float4* ko = kp + (bh * rows_out + r) * (2 * CPT);
    float4* vo = vp + (bh * rows_out + r) * (2 * CPT);
    for (int c = lane; c < 2 * CPT; c += 64) {
      float x[8];
      if (c < CPT) {
        unpack8(kb[src * CPT + c], x);
        if (r >= T) rope_apply(x, rope_cs(c, D, (float)by, (float)bx, fr));
        store8_f32(ko, c, x);
      } else {
        unpack8(vb[src * CPT + (c - CPT)], x);
        store8_f32(vo, c - CPT, x);
      }
    }
  }
}

// Haar detail energy of one 2x2 cell per thread, float64 with every
// operation in the written order (no contraction), channels in order.
__global__ __launch_bounds__(256) void dwt_kernel(const float* __restrict__ lat, float* __restrict__ energy,
                                                  int32_t* __restrict__ energy_q, int C, int Gh, int Gw) {
#pragma clang fp contract(off)
  int hw = Gw / 2, hh_ = Gh / 2;
  int64_t cells = (int64_t)hw * hh_;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cells;
       i += (int64_t)gridDim.x * blockDim.x) {
    int cy = (int)(i / hw), cx = (int)(i % hw);
    double E = 0.0;
    for (int ch = 0; ch < C; ++ch) {
      const float* base = lat + (int64_t)ch * Gh * Gw + (int64_t)(2 * cy) * Gw + 2 * cx;
      float2 top = *reinterpret_cast<const float2*>(base);
      float2 bot = *reinterpret_cast<const float2*>(base + Gw);
      double a = top.x, b = top.y, c = bot.x, d = bot.y;
      double lh = (((a - b) + c) - d) * 0.5;
      double hl = (((a + b) - c) - d) * 0.5;
      double hh = (((a - b) - c) + d) * 0.5;
      double l2 = lh * lh;
      double h2 = hl * hl;
      double s = l2 + h2;
      double d2 = hh * hh;
      E = E + (s + d2);
    }
    energy[i] = (float)E;
    double q = rint(E * 65536.0);
    if (q > 2147483647.0) q = 2147483647.0;
    energy_q[i] = (int32_t)q;
  }
}

int grid_for(int64_t work, int block = 256) {
  int64_t g = (work + block - 1) / block;
  const int64_t cap = 256LL * 2048;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(AREA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return AREA_OK;
}

}  // namespace

// 2-D launch for the per-(batch, head) kernels: x covers `per_bh` items of
// one (batch, head) in 256-thread blocks, y the (batch, head) pairs.
static dim3 grid_2d(int64_t per_bh, int64_t BH) {
  int64_t gx = (per_bh + 255) / 256;
  int64_t gy = BH;
  gx = std::max<int64_t>(1, std::min<int64_t>(gx, 1 << 16));
  gy = std::max<int64_t>(1, std::min<int64_t>(gy, 65535));
  return dim3((unsigned)gx, (unsigned)gy);
}

int launch_rope_table(void* tab, int Gh, int Gw, int D, float theta, float div, int* flags, int64_t n_flags,
                      stream_t s) {
  const int P = std::max(Gh, Gw), NF = D / 4;
  float2* t = (float2*)tab;
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(std::max<int64_t>((int64_t)P * NF, n_flags))), dim3(256), 0,
                     (hipStream_t)s, t, t + (size_t)P * NF, P, NF, div, make_inv_freq(D, theta), flags, n_flags);
  return check_launch("rope_table_kernel");
}

int launch_pool(const void* k, const void* v, void* kp, void* vp, int64_t BH, int T, int Gh, int Gw, int D,
                int f, int mode, unsigned long long seed, float theta, stream_t s) {
  InvFreq fr = make_inv_freq(D, theta);
  const int64_t rows_out = (int64_t)T + (int64_t)(Gh / f) * (Gw / f);
  if (mode == AREA_POOL_MEDOID) {
    if (rows_out > 0x7FFFFFFFLL) return fail(AREA_E_UNSUPPORTED, "too many pooled rows for the medoid grid");
    const dim3 grid((unsigned)rows_out, (unsigned)std::min<int64_t>(BH, 65535));
    if (D == 128)
      hipLaunchKernelGGL((pool_medoid_kernel<128>), grid, dim3(64), 0, (hipStream_t)s, (const uint4*)k,
                         (const uint4*)v, (float4*)kp, (float4*)vp, BH, Gh, Gw, f, T, fr);
    else
      hipLaunchKernelGGL((pool_medoid_kernel<64>), grid, dim3(64), 0, (hipStream_t)s, (const uint4*)k,
                         (const uint4*)v, (float4*)kp, (float4*)vp, BH, Gh, Gw, f, T, fr);
    return check_launch("pool_medoid_kernel");
  }
  const dim3 grid = grid_2d(rows_out * (D / 8), BH);
  if (D == 128)
    hipLaunchKernelGGL((pool_kernel<128>), grid, dim3(256), 0, (hipStream_t)s, (const uint4*)k, (const uint4*)v,
                       (float4*)kp, (float4*)vp, BH, Gh, Gw, f, mode, T, seed, fr);
  else
    hipLaunchKernelGGL((pool_kernel<64>), grid, dim3(256), 0, (hipStream_t)s, (const uint4*)k, (const uint4*)v,
                       (float4*)kp, (float4*)vp, BH, Gh, Gw, f, mode, T, seed, fr);
  return check_launch("pool_kernel");
}

int launch_dwt(const float* latent, float* energy, int32_t* energy_q, int C, int Gh, int Gw,
               stream_t s) {
  int64_t cells = (int64_t)(Gh / 2) * (Gw / 2);
  hipLaunchKernelGGL(dwt_kernel, dim3(grid_for(cells)), dim3(256), 0, (hipStream_t)s, latent, energy,
                     energy_q, C, Gh, Gw);
  return check_launch("dwt_kernel");
}

}  // namespace area
