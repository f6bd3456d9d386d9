// Flash-style attention on gfx950 for the AReA path: dense (full attention,
// Phase I coarse attention over pooled keys) and windowed (Phase II: Halo
// rectangle + bridge keys, tent-weighted blending of overlaps).
//
// Design (CDNA4, wave64):
//  * MFMA v_mfma_f32_32x32x16_f16 with fp32 accumulation for both Q K^T and
//    P V.  The operands (rotated Q and K, V, P) are IEEE fp16: the same MFMA
//    rate as bf16 with three more mantissa bits, so the bf16 rounding of the
//    output is the only coarse rounding on the path.
//  * The score tile is computed transposed, S^T = K Q^T, so that each lane
//    owns one query column: the softmax max/sum over keys is an in-lane
//    reduction plus one exchange with the partner lane (lane ^ 32).
//  * K rows are read in a permuted order so that the S^T accumulator
//    registers already form the bf16 B operand of O^T += V^T P^T; P never
//    leaves registers.
//  * K (row-major) and V (transposed) tiles of 64 keys are staged through
//    LDS, double-buffered, with the next tile's global loads in flight while
//    the current tile is computed; one barrier per tile.
//  * Online softmax in exp2 units with lazy rescaling: the running maximum
//    only moves when a new score exceeds it by more than 2^8, so the O
//    rescale is skipped on almost every tile.
//  * Work items are mapped XCD-aware: consecutive items (same head, same
//    window) land on the same XCD and share its L2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <string>

#include "area_internal.h"

namespace area {

namespace {

typedef unsigned short u16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = kAttnBN;
constexpr float kLazy = 8.0f;  // log2 headroom before the running max is moved

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(AREA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return AREA_OK;
}

struct AttnArgs {
  const u16* q;        // rotated queries, fp16 [BH][Nq][D]
  const u16* k;        // rotated keys, fp16 [BH][Nk][D]   (window mode: [BH][N][D])
  const u16* v;        // values, fp16 [BH][Nk][D]
  u16* out;            // [BH][Nq][D]
  int64_t BH;
  int Nq, Nk;          // dense mode sizes
  int n_qtiles;        // dense mode: query tiles per head
  int grid;            // launched work-groups (multiple of 8)
  float c;             // log2(e) / sqrt(D)
  // window mode
  const int32_t* plan;
  const int32_t* wsum;
  const int32_t* bridge;   // [BH][R] or null
  const int* items;        // [max_items][2] = (record, query tile)
  const int* n_items;
  const int* slot_off;     // per record: first slot of its query rect
  float* slots;            // [slot][BH][D] fp32 outputs of overlapped tokens
  int Gw, R;
  int64_t max_items;
};

__device__ inline u16 f2bf(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

// Unsigned division by a divisor d fixed per work item: q = umulhi(n, m)
// with m = ceil(2^32 / d) is exact whenever n * d < 2^32 (key slots and
// token indices here stay below 2^26 and d below 2^15); d = 1 is exact with
// m = 0 handled by the caller's select.
struct FastDiv {
  unsigned m;
  int d;
  __device__ static FastDiv make(int d) {
    FastDiv f;
    f.d = d;
    f.m = d > 1 ? 0xFFFFFFFFu / (unsigned)d + 1u : 0u;
    return f;
  }
  __device__ __attribute__((always_inline)) int div(int n) const {
    return d > 1 ? (int)__umulhi((unsigned)n, m) : n;
  }
};

struct WinRect {
  int qy0, qx0, qh, qw, ky0, kx0, kh, kw;
  FastDiv kwd, gwd;
};

// Token of key slot s of a window (Halo rectangle first, then the bridge
// list); bridge tokens inside the rectangle are invalid (already present).
__device__ __attribute__((always_inline)) inline int win_key(int s, const WinRect& r, int Gw, const int32_t* br,
                                                             int R, bool& valid) {
  int nrect = r.kh * r.kw;
  if (s < nrect) {
    valid = true;
    int yy = r.kwd.div(s);
    return (r.ky0 + yy) * Gw + r.kx0 + (s - yy * r.kw);
  }
  int j = s - nrect;
  if (j < R) {
    int tok = br[j];
    int y = r.gwd.div(tok), x = tok - y * Gw;
    valid = !(y >= r.ky0 && y < r.ky0 + r.kh && x >= r.kx0 && x < r.kx0 + r.kw);
    return tok;
  }
  valid = false;
  return 0;
}

// Per-thread staging of one 64-key tile: K rows as 16-byte chunks, V as
// VK consecutive keys x 8 channels (written transposed to LDS).
template <int D>
struct TileRegs {
  static constexpr int CPR = D / 8;
  static constexpr int K_CPT = kAttnBN * CPR / 256;
  static constexpr int VK = 8 * D / 256;
  u32x4 k[K_CPT];
  u32x4 v[VK];
};

template <bool WIN>
__device__ __attribute__((always_inline)) inline int key_token(int s, int nkv, const WinRect& r, int Gw,
                                                               const int32_t* br, int R, bool& valid) {
  if constexpr (WIN) {
    return win_key(s, r, Gw, br, R, valid);
  } else {
    valid = s < nkv;
    return valid ? s : nkv - 1;
  }
}

template <int D, bool WIN>
__device__ __attribute__((always_inline)) inline void load_tile(TileRegs<D>& t, int tile, int tid, int nkv,
                                                                const WinRect& r, int Gw, const int32_t* br, int R,
                                                                const u16* kbase, const u16* vbase) {
  constexpr int CPR = TileRegs<D>::CPR;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::K_CPT; ++i) {
    int c = tid + i * 256;
    int row = c / CPR, col = c - row * CPR;
    bool ok;
    int tok = key_token<WIN>(tile * kAttnBN + row, nkv, r, Gw, br, R, ok);
    t.k[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)tok * D + col * 8);
  }
  constexpr int KG = kAttnBN / TileRegs<D>::VK;  // key groups per tile
  int kg = tid % KG, dc = tid / KG;
#pragma unroll
  for (int q = 0; q < TileRegs<D>::VK; ++q) {
    bool ok;
    int tok = key_token<WIN>(tile * kAttnBN + kg * TileRegs<D>::VK + q, nkv, r, Gw, br, R, ok);
    t.v[q] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)tok * D + dc * 8);
  }
}

template <int D>
__device__ __attribute__((always_inline)) inline void store_tile(const TileRegs<D>& t, u16* ks, u16* vt, int tid) {
  constexpr int CPR = TileRegs<D>::CPR, VK = TileRegs<D>::VK;
  constexpr int KS = D + 8, VS = kAttnBN + 8;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::K_CPT; ++i) {
    int c = tid + i * 256;
    int row = c / CPR, col = c - row * CPR;
    // key row r lives in LDS row perm(r) (bits 2 and 3 swapped): MFMA row m
    // then reads LDS row m, so the 8 lanes served together by a 128-bit
    // read touch 8 consecutive rows, i.e. distinct banks
    int prow = (row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1);
    *reinterpret_cast<u32x4*>(ks + prow * KS + col * 8) = t.k[i];
  }
  constexpr int KG = kAttnBN / VK;
  int kg = tid % KG, dc = tid / KG;
#pragma unroll
  for (int jd = 0; jd < 8; ++jd) {
    unsigned e[VK];
#pragma unroll
    for (int q = 0; q < VK; ++q) {
      const unsigned w = t.v[q][jd >> 1];
      e[q] = (jd & 1) ? (w >> 16) : (w & 0xFFFFu);
    }
    u16* dst = vt + (dc * 8 + jd) * VS + kg * VK;
    if constexpr (VK == 4) {
      u32x2 pk = {e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
      *reinterpret_cast<u32x2*>(dst) = pk;
    } else {
      *reinterpret_cast<unsigned*>(dst) = e[0] | (e[1] << 16);
    }
  }
}

// S^T (keys x queries) of one tile for the wave's QG groups of 32 queries.
template <int D, int QG>
__device__ __attribute__((always_inline)) inline void tile_scores(f32x16 (&s)[QG][2], const u16* ks, int krow_perm,
                                                                  int hi, const f16x8 (&qf)[QG][D / 16]) {
  constexpr int KS = D + 8;
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[g][kb][i] = 0.0f;
  const u16* kr = ks + krow_perm * KS + 8 * hi;  // krow_perm: LDS row of MFMA row n
#pragma unroll
  for (int kd = 0; kd < D / 16; ++kd) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f16x8 af = *reinterpret_cast<const f16x8*>(kr + 32 * kb * KS + 16 * kd);
#pragma unroll
      for (int g = 0; g < QG; ++g) s[g][kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, qf[g][kd], s[g][kb], 0, 0, 0);
    }
  }
}

// O^T += V^T P^T for one tile.
template <int D, int QG>
__device__ __attribute__((always_inline)) inline void tile_pv(f32x16 (&o)[QG][D / 32], const u16* vt, int n, int hi,
                                                              const f16x8 (&pf)[QG][4]) {
  constexpr int VS = kAttnBN + 8;
  const u16* vr = vt + n * VS + 8 * hi;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      f16x8 af = *reinterpret_cast<const f16x8*>(vr + 32 * db * VS + 16 * ks);
#pragma unroll
      for (int g = 0; g < QG; ++g) o[g][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, pf[g][ks], o[g][db], 0, 0, 0);
    }
  }
}

// Keys of the tile that are not valid (tail of the key set, bridge tokens
// already inside the Halo rectangle) get a -inf score.  vm holds one bit per
// key of the tile; S^T register 8*jj + i of block kb is key
// 32 kb + 16 jj + 8 hi + i.
template <int QG>
__device__ __attribute__((always_inline)) inline void mask_scores(f32x16 (&s)[QG][2], uint64_t vm, int hi) {
  const uint32_t lm0 = (uint32_t)(vm >> (8 * hi));
  const uint32_t lm1 = (uint32_t)(vm >> (32 + 8 * hi));
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t bits = kb ? lm1 : lm0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        int bit = 16 * (i >> 3) + (i & 7);
        s[g][kb][i] = ((bits >> bit) & 1u) ? s[g][kb][i] : -INFINITY;
      }
    }
}

// Combine a value with the one held by the lane 32 apart (the other half of
// the same query column), without a trip through LDS.
__device__ __attribute__((always_inline)) inline float pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __attribute__((always_inline)) inline float pair_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online softmax of one tile (exp2 units, lazy maximum): P^T in fp16,
// running sums updated, per-group rescale factors of O returned.
template <int QG>
__device__ __attribute__((always_inline)) inline void tile_softmax(const f32x16 (&s)[QG][2], float c,
                                                                   float (&m_run)[QG], float (&l_run)[QG],
                                                                   float (&alpha)[QG], f16x8 (&pf)[QG][4]) {
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    float mx = fmaxf(s[g][0][0], s[g][0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[g][kb][i]);
    mx = pair_max(mx);
    const float mc = mx * c;
    const float m_new = mc > m_run[g] + kLazy ? mc : m_run[g];
    alpha[g] = __builtin_amdgcn_exp2f(m_run[g] - m_new);
    m_run[g] = m_new;
    const float negm = -m_new;
    float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f16x8 pv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[g][kb][8 * hh + i], c, negm));
          if (i & 1) ls1 += p; else ls0 += p;
          pv[i] = (_Float16)p;
        }
        pf[g][2 * kb + hh] = pv;
      }
    }
    l_run[g] = l_run[g] * alpha[g] + (ls0 + ls1);
  }
}

template <int D, bool WIN>
__global__ __launch_bounds__(256, 2) void attn_kernel(const AttnArgs a) {
  constexpr int QG = kAttnQG;     // 32-query groups per wave
  constexpr int BM = kAttnBM;     // 4 waves x QG groups x 32 queries
  constexpr int KD = D / 16;
  constexpr int DB = D / 32;
  constexpr int KS = D + 8;
  constexpr int VS = BN + 8;
  constexpr int K_ELEMS = BN * KS;
  constexpr int V_ELEMS = D * VS;
  constexpr int STAGE = K_ELEMS + V_ELEMS;
  static_assert(BM == 4 * 32 * QG, "query tile");

  // two LDS stages: the tile being multiplied and the tile being written
  __shared__ __attribute__((aligned(16))) u16 smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hi = lane >> 5;

  // ---- work item (XCD-aware order: logical ids are contiguous per XCD)
  const int pid = blockIdx.x;
  const int64_t L = (int64_t)(pid & 7) * (a.grid >> 3) + (pid >> 3);
  int64_t bh;
  int qtile = 0, rec = 0;
  WinRect r = {};
  int nq, nkv;
  if constexpr (WIN) {
    bh = L / a.max_items;
    int64_t it = L - bh * a.max_items;
    if (bh >= a.BH || it >= *a.n_items) return;
    rec = a.items[2 * it];
    qtile = a.items[2 * it + 1];
    const int32_t* rp = a.plan + AREA_PLAN_HEADER + AREA_PLAN_REC * rec;
    r.qy0 = rp[0]; r.qx0 = rp[1]; r.qh = rp[2]; r.qw = rp[3];
    r.ky0 = rp[4]; r.kx0 = rp[5]; r.kh = rp[6]; r.kw = rp[7];
    r.kwd = FastDiv::make(r.kw);
    r.gwd = FastDiv::make(a.Gw);
    nq = r.qh * r.qw;
    nkv = r.kh * r.kw + a.R;
  } else {
    bh = L / a.n_qtiles;
    qtile = (int)(L - bh * a.n_qtiles);
    if (bh >= a.BH) return;
    nq = a.Nq;
    nkv = a.Nk;
  }
  const int32_t* br = (WIN && a.R > 0) ? a.bridge + bh * a.R : nullptr;
  const int64_t kv_rows = WIN ? (int64_t)a.Nq : (int64_t)a.Nk;
  const u16* kbase = a.k + bh * kv_rows * D;
  const u16* vbase = a.v + bh * kv_rows * D;
  const u16* qbase = a.q + bh * (int64_t)a.Nq * D;

  // ---- queries of this lane
  int qtok[QG];
  bool qvalid[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    int t = qtile * BM + wave * 32 * QG + 32 * g + n;
    qvalid[g] = t < nq;
    if constexpr (WIN) {
      int yy = qvalid[g] ? t / r.qw : 0;
      int xx = qvalid[g] ? t - yy * r.qw : 0;
      qtok[g] = (r.qy0 + yy) * a.Gw + r.qx0 + xx;
    } else {
      qtok[g] = qvalid[g] ? t : 0;
    }
  }
  f16x8 qf[QG][KD];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const f16x8* qrow = reinterpret_cast<const f16x8*>(qbase + (int64_t)qtok[g] * D);
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) qf[g][kd] = qrow[2 * kd + hi];
  }

  const int nt = (nkv + BN - 1) / BN;
  const float c = a.c;
  // MFMA row n of the score tile is key perm(n) (bits 2 and 3 swapped), so
  // that S^T registers 8*jj + i of block kb hold key 32 kb + 16 jj + 8 hi + i;
  // store_tile already placed key perm(n) in LDS row n.
  const int krow_perm = n;

  f32x16 o[QG][DB];
  float m_run[QG], l_run[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[g][db][i] = 0.0f;
  }

  // ---- prologue: tile 0 to LDS, tile 1 in flight
  TileRegs<D> tr;
  load_tile<D, WIN>(tr, 0, tid, nkv, r, a.Gw, br, a.R, kbase, vbase);
  store_tile<D>(tr, smem, smem + K_ELEMS, tid);
  load_tile<D, WIN>(tr, 1, tid, nkv, r, a.Gw, br, a.R, kbase, vbase);
  __syncthreads();

  for (int j = 0; j < nt; ++j) {
    u16* ks = smem + (j & 1) * STAGE;
    u16* vt = ks + K_ELEMS;
    uint64_t vm;
    {
      bool ok;
      (void)key_token<WIN>(j * BN + lane, nkv, r, a.Gw, br, a.R, ok);
      vm = __ballot(ok);
    }
    f32x16 s[QG][2];
    tile_scores<D, QG>(s, ks, krow_perm, hi, qf);
    if (vm != ~0ull) mask_scores<QG>(s, vm, hi);
    float alpha[QG];
    f16x8 pf[QG][4];
    tile_softmax<QG>(s, c, m_run, l_run, alpha, pf);
    bool resc = false;
#pragma unroll
    for (int g = 0; g < QG; ++g) resc |= alpha[g] != 1.0f;
    if (__any(resc)) {
#pragma unroll
      for (int g = 0; g < QG; ++g)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[g][db][i] *= alpha[g];
    }
    tile_pv<D, QG>(o, vt, n, hi, pf);
    if (j + 1 < nt) {
      u16* ks2 = smem + ((j + 1) & 1) * STAGE;
      store_tile<D>(tr, ks2, ks2 + K_ELEMS, tid);
      load_tile<D, WIN>(tr, j + 2, tid, nkv, r, a.Gw, br, a.R, kbase, vbase);
    }
    __syncthreads();
  }

  // ---- epilogue: normalise and write
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    float lt = pair_sum(l_run[g]);
    float inv = 1.0f / lt;
    if (!qvalid[g]) continue;
    if constexpr (WIN) {
      int t = qtile * BM + wave * 32 * QG + 32 * g + n;
      int uy = t / r.qw, ux = t - (t / r.qw) * r.qw;
      int wt = min(uy + 1, r.qh - uy) * min(ux + 1, r.qw - ux);
      int tok = qtok[g];
      if (a.wsum[tok] == wt) {
        u16* orow = a.out + (bh * (int64_t)a.Nq + tok) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            int d = 32 * db + 8 * q4 + 4 * hi;
            uint2 pk;
            pk.x = (unsigned)f2bf(o[g][db][4 * q4 + 0] * inv) | ((unsigned)f2bf(o[g][db][4 * q4 + 1] * inv) << 16);
            pk.y = (unsigned)f2bf(o[g][db][4 * q4 + 2] * inv) | ((unsigned)f2bf(o[g][db][4 * q4 + 3] * inv) << 16);
            *reinterpret_cast<uint2*>(orow + d) = pk;
          }
      } else {
        float* srow = a.slots + ((int64_t)(a.slot_off[rec] + t) * a.BH + bh) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            int d = 32 * db + 8 * q4 + 4 * hi;
            float4 v4 = make_float4(o[g][db][4 * q4 + 0] * inv, o[g][db][4 * q4 + 1] * inv,
                                    o[g][db][4 * q4 + 2] * inv, o[g][db][4 * q4 + 3] * inv);
            *reinterpret_cast<float4*>(srow + d) = v4;
          }
      }
    } else {
      u16* orow = a.out + (bh * (int64_t)a.Nq + qtok[g]) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          int d = 32 * db + 8 * q4 + 4 * hi;
          uint2 pk;
          pk.x = (unsigned)f2bf(o[g][db][4 * q4 + 0] * inv) | ((unsigned)f2bf(o[g][db][4 * q4 + 1] * inv) << 16);
          pk.y = (unsigned)f2bf(o[g][db][4 * q4 + 2] * inv) | ((unsigned)f2bf(o[g][db][4 * q4 + 3] * inv) << 16);
          *reinterpret_cast<uint2*>(orow + d) = pk;
        }
    }
  }
}

// ------------------------------------------------------------ work list --
// Items workspace: [0] n_items, then slot_off[max_windows],
// rec_start[n_base], items[max_items][2].
struct ItemsWs {
  int* n_items;
  int* slot_off;
  int* rec_start;
  int* items;
};

ItemsWs make_items_ws(void* ws, int max_windows, int n_base) {
  ItemsWs w;
  char* p = (char*)ws;
  w.n_items = (int*)p;
  p += align_up(sizeof(int));
  w.slot_off = (int*)p;
  p += align_up(sizeof(int) * (max_windows > 0 ? max_windows : 1));
  w.rec_start = (int*)p;
  p += align_up(sizeof(int) * (n_base > 0 ? n_base : 1));
  w.items = (int*)p;
  return w;
}

// One block: slot offsets (prefix of query areas in record order), the
// first record of every base window, and the (record, query tile) list with
// whole windows first and quadrants after (largest key sets first).
__global__ __launch_bounds__(256) void items_kernel(const int32_t* __restrict__ plan, ItemsWs w, int BM,
                                                    int max_windows, int64_t max_items) {
  __shared__ int s_item_off[4 * kMaxAxisWindows * kMaxAxisWindows];
  int nwin = plan[AREA_PH_NWIN];
  if (nwin > max_windows) nwin = max_windows;
  if (threadIdx.x == 0) {
    int qs = 0, it = 0;
    for (int pass = 0; pass < 2; ++pass) {
      for (int i = 0; i < nwin; ++i) {
        const int32_t* rp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * i;
        bool quad = rp[9] >= 0;
        if ((pass == 0) == quad) continue;
        s_item_off[i] = it;
        it += (rp[2] * rp[3] + BM - 1) / BM;
      }
    }
    for (int i = 0; i < nwin; ++i) {
      const int32_t* rp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * i;
      w.slot_off[i] = qs;
      qs += rp[2] * rp[3];
      if (rp[9] <= 0) w.rec_start[rp[8]] = i;
    }
    if (it > max_items) it = (int)max_items;
    *w.n_items = it;
  }
  __syncthreads();
  for (int i = 0; i < nwin; ++i) {
    const int32_t* rp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * i;
    int nt = (rp[2] * rp[3] + BM - 1) / BM;
    for (int t = threadIdx.x; t < nt; t += blockDim.x) {
      int idx = s_item_off[i] + t;
      if (idx < max_items) {
        w.items[2 * idx] = i;
        w.items[2 * idx + 1] = t;
      }
    }
  }
}

struct BlendArgs {
  int Gh, Gw, D, ny, nx, Ly, Lx;
  int64_t BH;
  int ys[kMaxAxisWindows], xs[kMaxAxisWindows];
};

constexpr int kBlendTok = 16;
constexpr int kMaxCover = 8;

__device__ inline int tent_w(int u, int L) { return min(u + 1, L - u); }

// Tokens covered by more than one window: out = sum_w wt_w * O_w / wsum,
// windows in record order.
__global__ __launch_bounds__(256) void blend_kernel(BlendArgs b, const int32_t* __restrict__ plan,
                                                    const int* __restrict__ rec_start, const int* __restrict__ slot_off,
                                                    const int32_t* __restrict__ wsum, const float* __restrict__ slots,
                                                    u16* __restrict__ out) {
  __shared__ int s_slot[kMaxCover * kMaxCover];
  __shared__ float s_wt[kMaxCover * kMaxCover];
  __shared__ int s_cnt;
  int64_t N = (int64_t)b.Gh * b.Gw;
  int D4 = b.D / 4;
  for (int k = 0; k < kBlendTok; ++k) {
    int64_t p = (int64_t)blockIdx.x * kBlendTok + k;
    if (p >= N) break;
    int y = (int)(p / b.Gw), x = (int)(p % b.Gw);
    if (threadIdx.x == 0) {
      int iy[kMaxCover], ix[kMaxCover], cy = 0, cx = 0;
      for (int i = 0; i < b.ny; ++i)
        if (y >= b.ys[i] && y < b.ys[i] + b.Ly && cy < kMaxCover) iy[cy++] = i;
      for (int j = 0; j < b.nx; ++j)
        if (x >= b.xs[j] && x < b.xs[j] + b.Lx && cx < kMaxCover) ix[cx++] = j;
      int cnt = 0;
      if (cy * cx > 1) {
        for (int a = 0; a < cy; ++a)
          for (int c = 0; c < cx; ++c) {
            int r0 = rec_start[iy[a] * b.nx + ix[c]];
            int rr = r0;
            const int32_t* rp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * r0;
            if (rp[9] >= 0) {
              // split window: pick the quadrant holding (y, x)
              for (int qd = 0; qd < 4; ++qd) {
                const int32_t* qp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * (r0 + qd);
                if (y >= qp[0] && y < qp[0] + qp[2] && x >= qp[1] && x < qp[1] + qp[3]) rr = r0 + qd;
              }
            }
            const int32_t* wp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * rr;
            int uy = y - wp[0], ux = x - wp[1];
            s_wt[cnt] = (float)(tent_w(uy, wp[2]) * tent_w(ux, wp[3]));
            s_slot[cnt] = slot_off[rr] + uy * wp[3] + ux;
            ++cnt;
          }
      }
      s_cnt = cnt;
    }
    __syncthreads();
    int cnt = s_cnt;
    if (cnt > 1) {
      float inv = 1.0f / (float)wsum[p];
      for (int e = threadIdx.x; e < b.BH * D4; e += blockDim.x) {
        int64_t bh = e / D4;
        int d4 = e - (int)bh * D4;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int i = 0; i < cnt; ++i) {
          float4 v = *reinterpret_cast<const float4*>(slots + ((int64_t)s_slot[i] * b.BH + bh) * b.D + 4 * d4);
          float wgt = s_wt[i];
          acc.x += wgt * v.x;
          acc.y += wgt * v.y;
          acc.z += wgt * v.z;
          acc.w += wgt * v.w;
        }
        uint2 pk;
        pk.x = (unsigned)f2bf(acc.x * inv) | ((unsigned)f2bf(acc.y * inv) << 16);
        pk.y = (unsigned)f2bf(acc.z * inv) | ((unsigned)f2bf(acc.w * inv) << 16);
        *reinterpret_cast<uint2*>(out + (bh * N + p) * b.D + 4 * d4) = pk;
      }
    }
    __syncthreads();
  }
}

template <bool WIN>
int launch_attn(const AttnArgs& a, int D, int64_t work, hipStream_t st) {
  AttnArgs b = a;
  int64_t g = (work + 7) / 8 * 8;
  if (g > 0x7FFFFFFFLL) return fail(AREA_E_UNSUPPORTED, "attention grid too large");
  b.grid = (int)g;
  dim3 grid((unsigned)b.grid);
  AttnEvents ev = attn_events();
  if (ev.begin) {
    hipError_t e = hipEventRecord((hipEvent_t)ev.begin, st);
    if (e != hipSuccess) return fail(AREA_E_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
  }
  if (D == 128)
    hipLaunchKernelGGL((attn_kernel<128, WIN>), grid, dim3(256), 0, st, b);
  else
    hipLaunchKernelGGL((attn_kernel<64, WIN>), grid, dim3(256), 0, st, b);
  int rc = check_launch(WIN ? "attn_kernel<window>" : "attn_kernel<dense>");
  if (rc) return rc;
  if (ev.end) {
    hipError_t e = hipEventRecord((hipEvent_t)ev.end, st);
    if (e != hipSuccess) return fail(AREA_E_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
  }
  return AREA_OK;
}

}  // namespace

int launch_dense_attn(const void* q_rot, const void* k_rot, const void* v, void* out, int64_t BH, int Nq,
                      int Nk, int D, stream_t s) {
  AttnArgs a = {};
  a.q = (const u16*)q_rot;
  a.k = (const u16*)k_rot;
  a.v = (const u16*)v;
  a.out = (u16*)out;
  a.BH = BH;
  a.Nq = Nq;
  a.Nk = Nk;
  a.n_qtiles = (Nq + kAttnBM - 1) / kAttnBM;
  a.c = (float)(1.4426950408889634 / std::sqrt((double)D));
  return launch_attn<false>(a, D, (int64_t)a.n_qtiles * BH, (hipStream_t)s);
}

size_t window_items_ws_bytes(int max_windows, int64_t max_items, int n_base) {
  return align_up(sizeof(int)) + align_up(sizeof(int) * (max_windows > 0 ? max_windows : 1)) +
         align_up(sizeof(int) * (n_base > 0 ? n_base : 1)) + align_up(sizeof(int) * 2 * (max_items > 0 ? max_items : 1));
}

int launch_window_attn(const WindowAttnArgs& w, const int32_t* plan, const int32_t* wsum, const int32_t* bridge_idx,
                       const void* q_rot, const void* k_rot, const void* v, void* out, void* items_ws, float* slots,
                       stream_t s) {
  hipStream_t st = (hipStream_t)s;
  int n_base = w.ny * w.nx;
  ItemsWs iw = make_items_ws(items_ws, w.max_windows, n_base);
  hipLaunchKernelGGL(items_kernel, dim3(1), dim3(256), 0, st, plan, iw, kAttnBM, w.max_windows, w.max_items);
  int rc = check_launch("items_kernel");
  if (rc) return rc;
  AttnArgs a = {};
  a.q = (const u16*)q_rot;
  a.k = (const u16*)k_rot;
  a.v = (const u16*)v;
  a.out = (u16*)out;
  a.BH = w.BH;
  a.Nq = w.Gh * w.Gw;
  a.Nk = w.Gh * w.Gw;
  a.c = (float)(1.4426950408889634 / std::sqrt((double)w.D));
  a.plan = plan;
  a.wsum = wsum;
  a.bridge = bridge_idx;
  a.items = iw.items;
  a.n_items = iw.n_items;
  a.slot_off = iw.slot_off;
  a.slots = slots;
  a.Gw = w.Gw;
  a.R = bridge_idx ? w.R : 0;
  a.max_items = w.max_items;
  rc = launch_attn<true>(a, w.D, w.max_items * w.BH, st);
  if (rc) return rc;
  BlendArgs b;
  b.Gh = w.Gh;
  b.Gw = w.Gw;
  b.D = w.D;
  b.ny = w.ny;
  b.nx = w.nx;
  b.Ly = w.Ly;
  b.Lx = w.Lx;
  b.BH = w.BH;
  for (int i = 0; i < kMaxAxisWindows; ++i) {
    b.ys[i] = w.ys[i];
    b.xs[i] = w.xs[i];
  }
  int64_t N = (int64_t)w.Gh * w.Gw;
  hipLaunchKernelGGL(blend_kernel, dim3((unsigned)((N + kBlendTok - 1) / kBlendTok)), dim3(256), 0, st, b, plan,
                     (const int*)iw.rec_start, (const int*)iw.slot_off, wsum, (const float*)slots, (u16*)out);
  return check_launch("blend_kernel");
}

}  // namespace area
