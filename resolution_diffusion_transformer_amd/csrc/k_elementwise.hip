// Bandwidth-bound kernels of the AReA path on gfx950: two-axis RoPE
// rotation, f x f key/value pooling with RoPE at coarse positions, and the
// Haar detail-energy map.
#include <hip/hip_runtime.h>

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

__device__ inline float bf16_to_f32(unsigned short h) { return __uint_as_float(((unsigned)h) << 16); }

// float -> bfloat16, round to nearest even (inputs are finite).
__device__ inline unsigned short f32_to_bf16(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

__device__ inline void unpack8(const uint4& r, float* x) {
  const unsigned w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// float -> IEEE half, round to nearest even.
__device__ inline unsigned short f32_to_f16(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(unsigned short, h);
}

__device__ inline uint4 pack8_f16(const float* x) {
  unsigned w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (unsigned)f32_to_f16(x[2 * i]) | ((unsigned)f32_to_f16(x[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ inline uint4 pack8(const float* x) {
  unsigned w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (unsigned)f32_to_bf16(x[2 * i]) | ((unsigned)f32_to_bf16(x[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Rotate the 8 channels [8c, 8c+8) of one token at grid position (py, px).
// Channels below D/2 follow the row, the others the column; pair
// (2k, 2k+1) of an axis half turns by pos * inv_freq[k].
__device__ inline void rope8(float* x, int c, int D, float py, float px, const InvFreq& f) {
  int d0 = 8 * c;
  int half = D / 2;
  float pos = d0 < half ? py : px;
  int k0 = (d0 % half) / 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float s, co;
    sincosf(pos * f.v[k0 + j], &s, &co);
    float a = x[2 * j], b = x[2 * j + 1];
    x[2 * j] = a * co - b * s;
    x[2 * j + 1] = a * s + b * co;
  }
}

// Attention operand preparation, one thread per 8 channels of a token of
// the joint sequence (T text tokens, then the image grid):
//   qo = RoPE(q) and ko = RoPE(k) at positions (row / div, col / div) for
// image tokens and (0, 0) -- no rotation -- for text tokens, vo = v, all
// written as IEEE fp16 (the MFMA operand type of the attention kernels;
// bf16 -> fp16 is exact in fp16's normal range and the rotated values keep
// three more mantissa bits than bf16 would).  k / v may be null to skip them.
__global__ __launch_bounds__(256) void prep_kernel(const uint4* __restrict__ q, const uint4* __restrict__ k,
                                                   const uint4* __restrict__ v, uint4* __restrict__ qo,
                                                   uint4* __restrict__ ko, uint4* __restrict__ vo,
                                                   int64_t total_chunks, int L, int T, int Gw, int D, float div,
                                                   InvFreq f) {
  int cpt = D / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks;
       i += (int64_t)gridDim.x * blockDim.x) {
    int c = (int)(i % cpt);
    int n = (int)((i / cpt) % L) - T;
    float py = n < 0 ? 0.0f : (float)(n / Gw) / div;
    float px = n < 0 ? 0.0f : (float)(n % Gw) / div;
    float x[8];
    unpack8(q[i], x);
    rope8(x, c, D, py, px, f);
    qo[i] = pack8_f16(x);
    if (k) {
      unpack8(k[i], x);
      rope8(x, c, D, py, px, f);
      ko[i] = pack8_f16(x);
    }
    if (v) {
      unpack8(v[i], x);
      vo[i] = pack8_f16(x);
    }
  }
}

// Pooled keys/values: one thread per (batch*head, output row, 8 channels).
// The first T output rows are the text keys and values, copied unpooled and
// unrotated (text sits at position (0, 0)).  For a pooled row, mean mode
// sums the block's f*f tokens in fp32 (block rows in order, then columns)
// and divides by f*f; centre mode takes token (f/2, f/2) of the block.  Keys
// are then rotated at the coarse position (by, bx); values are not rotated.
// One rounding at the end, to fp16 (the attention MFMA operand type).
__global__ __launch_bounds__(256) void pool_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                   uint4* __restrict__ kp, uint4* __restrict__ vp,
                                                   int64_t total_chunks, int Gh, int Gw, int D, int f,
                                                   int mode, int T, InvFreq fr) {
  int cpt = D / 8;
  int Wp = Gw / f, Hp = Gh / f;
  int64_t Np = (int64_t)Hp * Wp;
  int64_t L = T + (int64_t)Gh * Gw;   // input rows per (batch, head)
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks;
       i += (int64_t)gridDim.x * blockDim.x) {
    int c = (int)(i % cpt);
    int64_t t = i / cpt;
    int64_t r = t % (T + Np);
    int64_t bh = t / (T + Np);
    float ks[8], vs[8];
    if (r < T) {
      unpack8(k[(bh * L + r) * cpt + c], ks);
      unpack8(v[(bh * L + r) * cpt + c], vs);
      kp[i] = pack8_f16(ks);
      vp[i] = pack8_f16(vs);
      continue;
    }
    int np = (int)(r - T);
    int by = np / Wp, bx = np % Wp;
    const uint4* kb = k + (bh * L + T) * cpt + c;
    const uint4* vb = v + (bh * L + T) * cpt + c;
    if (mode == AREA_POOL_CENTER) {
      int64_t n = (int64_t)(by * f + f / 2) * Gw + (bx * f + f / 2);
      unpack8(kb[n * cpt], ks);
      unpack8(vb[n * cpt], vs);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) ks[j] = vs[j] = 0.0f;
      for (int dy = 0; dy < f; ++dy) {
        int64_t row = (int64_t)(by * f + dy) * Gw + bx * f;
        for (int dx = 0; dx < f; ++dx) {
          float a[8], b[8];
          unpack8(kb[(row + dx) * cpt], a);
          unpack8(vb[(row + dx) * cpt], b);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            ks[j] += a[j];
            vs[j] += b[j];
          }
        }
      }
      float inv = (float)(f * f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ks[j] = ks[j] / inv;
        vs[j] = vs[j] / inv;
      }
    }
    rope8(ks, c, D, (float)by, (float)bx, fr);
    kp[i] = pack8_f16(ks);
    vp[i] = pack8_f16(vs);
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

int launch_prep(const void* q, const void* k, const void* v, void* qo, void* ko, void* vo, int64_t BH,
                int T, int Gh, int Gw, int D, float theta, float div, stream_t s) {
  const int L = T + Gh * Gw;
  int64_t total = BH * (int64_t)L * (D / 8);
  InvFreq f = make_inv_freq(D, theta);
  hipLaunchKernelGGL(prep_kernel, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)s, (const uint4*)q,
                     (const uint4*)k, (const uint4*)v, (uint4*)qo, (uint4*)ko, (uint4*)vo, total, L, T, Gw,
                     D, div, f);
  return check_launch("prep_kernel");
}

int launch_pool(const void* k, const void* v, void* kp, void* vp, int64_t BH, int T, int Gh, int Gw, int D,
                int f, int mode, float theta, stream_t s) {
  int64_t total = BH * ((int64_t)T + (int64_t)(Gh / f) * (Gw / f)) * (D / 8);
  InvFreq fr = make_inv_freq(D, theta);
  hipLaunchKernelGGL(pool_kernel, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)s,
                     (const uint4*)k, (const uint4*)v, (uint4*)kp, (uint4*)vp, total, Gh, Gw, D, f,
                     mode, T, fr);
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
