// Flash-style attention on gfx950 for the AReA path: full attention, Phase I
// coarse attention over pooled keys, and Phase II windowed attention (Halo
// rectangle + global-KV bridge, tent-weighted blending of overlaps).
//
// Design (CDNA4, wave64):
//  * One attention kernel for every mode.  Its key/value set is always a
//    contiguous run of fp16 K rows plus fp16 V^T tiles of 64 keys, each tile
//    with a power-of-two exponent: full and coarse attention convert their
//    keys once per call (kv_tiles_kernel), windowed attention first gathers
//    each window's keys (Halo rectangle, then the bridge tokens outside it,
//    compacted, then the text keys; turned by RoPE on the way) with a
//    bandwidth-bound kernel, so no index math or transposition remains in
//    the MFMA loop.
//  * Queries are read once per work item as bf16 and turned by RoPE through
//    a (cos, sin) table into fp16 registers, so no rotated copy of Q is
//    written.
//  * MFMA v_mfma_f32_32x32x16_f16 with fp32 accumulation for Q K^T and P V.
//    fp16 operands run at the bf16 rate with three more mantissa bits, so the
//    bf16 rounding of the output is the only coarse rounding on the path.
//  * Scores are computed transposed, S^T = K Q^T: each lane owns one query
//    column, the softmax max/sum over keys is an in-lane reduction plus one
//    v_permlane32_swap with the partner lane.  K rows sit in LDS in the
//    order that makes the S^T accumulator registers the fp16 B operand of
//    O^T += V^T P^T, so P never leaves registers.
//  * K and V^T tiles reach LDS by global->LDS DMA (buffer_load ... lds, no
//    register staging), double-buffered and one barrier per tile.  Rows are
//    unpadded and the 16-byte chunks XOR-swizzled by row, so the 128-bit
//    MFMA operand reads are bank-conflict free.
//  * Each wave runs a two-phase software pipeline over key tiles: the
//    matrix cores compute the scores of tile j+1 while the VALU turns the
//    scores of tile j into P (exp2, fp16) and sums it, then they compute
//    O += P V for tile j.
//    sched_group_barrier interleaves the two instruction streams, so the
//    softmax runs in the shadow of the MFMAs instead of after them.
//  * Eight waves of 32 queries (256 queries per work-group) use 256
//    VGPRs: one work-group per CU, two waves per SIMD, and one K/V tile DMA
//    serves 256 queries.  In the last, partial query tile of a window, waves
//    with no query left only take their share of the DMAs and barriers, so
//    the working waves have their SIMDs to themselves.
//  * Online softmax in exp2 units with lazy rescaling: the running maximum
//    only moves when a lane's P sum over a tile exceeds 2^8, which bounds
//    every P it holds; it then moves to the tile's maximum and P is
//    recomputed.  No per-tile maximum is taken otherwise.
//    The queries carry log2(e)/sqrt(D) and each score accumulator starts
//    from -m, so the MFMA emits scores relative to the maximum and the
//    softmax is one exp2 and half a packed conversion per score; the exp2
//    go to the transcendental issue class, paired two per MFMA.
//  * Persistent work-groups, one per CU, claim work items from per-XCD
//    counters: consecutive items (same head, same window) run on the same
//    XCD and share its L2, and the next item's first tile DMAs are issued
//    before the current item's epilogue.
//  * Queries, key tiles or value tiles outside fp16's comfortable range
//    carry nonzero exponents; the items that meet one are listed by the
//    plain kernel and run by a second kernel that undoes the scales in fp32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <string>
#include <type_traits>

#include "area_internal.h"

namespace area {

namespace {

typedef unsigned short u16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = kAttnBN;
// A lane's P sum over a tile above this (2^8) moves the running maximum.
constexpr float kPsumMax = 256.0f;
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + vmcnt[5:4] at bits 15:14,
// expcnt[6:4], lgkmcnt[11:8]): wait for every vector memory operation.
constexpr int kVmcnt0 = 0x0F70;

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(AREA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return AREA_OK;
}

__device__ inline u16 f2bf(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

// Two-axis RoPE of one 16-byte chunk (8 bf16 channels, 4 rotation pairs)
// into fp16: c01, c23 hold the chunk's four (cos, sin) pairs, interleaved.
// Pair (a, b) becomes (a cos - b sin, a sin + b cos) times `scale`; the
// largest magnitude of these values is folded into `mx`, and with e != 0
// they are further scaled by 2^-e before rounding to nearest.
__device__ inline u32x4 rope8_f16_max(const u32x4 raw, const float4 c01, const float4 c23, const float scale,
                                      float& mx, const int e = 0) {
  const float co[4] = {c01.x, c01.z, c23.x, c23.z};
  const float sn[4] = {c01.y, c01.w, c23.y, c23.w};
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = __uint_as_float(raw[j] << 16), b = __uint_as_float(raw[j] & 0xFFFF0000u);
    float y0 = (a * co[j] - b * sn[j]) * scale;
    float y1 = (a * sn[j] + b * co[j]) * scale;
    mx = fmaxf(mx, fmaxf(fabsf(y0), fabsf(y1)));
    if (e != 0) {
      y0 = ldexpf(y0, -e);
      y1 = ldexpf(y1, -e);
    }
    const _Float16 x0 = (_Float16)y0, x1 = (_Float16)y1;
    r[j] = (unsigned)__builtin_bit_cast(u16, x0) | ((unsigned)__builtin_bit_cast(u16, x1) << 16);
  }
  return r;
}

// ------------------------------------------------------- operand range --
// fp16 holds magnitudes up to 65504 (normal down to 2^-14), less than bf16
// inputs can reach.  Every 64-key tile of K (and of V) is therefore stored
// as x * 2^-e with its own power-of-two exponent e, and every query row
// likewise: e = 0 while the block's largest magnitude m lies in
// [2^-8, 2^15) (or m is 0, subnormal, infinite or NaN), otherwise
// m * 2^-e lands in [2^13, 2^14).  Power-of-two scaling is exact, so
// in-range data is stored exactly as before; the attention kernel undoes
// nonzero exponents in fp32 (see its "scaled" loop).
__device__ inline int operand_exponent(float m) {
  const int eb = (int)((__float_as_uint(m) >> 23) & 0xFFu) - 127;  // floor(log2 m) for normal m
  if (eb == 128 || eb == -127) return 0;
  return (eb >= 15 || eb < -8) ? eb - 13 : 0;
}

// Largest magnitude over the 256 threads of a work-group (non-negative
// inputs; `red` holds 4 floats).
__device__ inline float block_max4(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

__device__ inline float maxabs8(const float* x, float m) {
#pragma unroll
  for (int i = 0; i < 8; i += 2) m = fmaxf(m, fmaxf(fabsf(x[i]), fabsf(x[i + 1])));
  return m;
}

__device__ inline void bf8_to_f32(const u32x4 raw, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(raw[i] << 16);
    x[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
  }
}

// x * 2^-e rounded to fp16 (to nearest even), 8 values into 16 bytes.
__device__ inline u32x4 f16x8_scaled(const float* x, int e) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 a = (_Float16)ldexpf(x[2 * i], -e), b = (_Float16)ldexpf(x[2 * i + 1], -e);
    r[i] = (unsigned)__builtin_bit_cast(u16, a) | ((unsigned)__builtin_bit_cast(u16, b) << 16);
  }
  return r;
}

// Two-axis RoPE of 8 channels in fp32: pair (a, b) -> (a cos - b sin,
// a sin + b cos) with the chunk's four (cos, sin) pairs from the [P][D/4]
// table row `cs`.
__device__ inline void rope8_f32(float* x, const float4* cs) {
  const float4 c01 = cs[0], c23 = cs[1];
  const float co[4] = {c01.x, c01.z, c23.x, c23.z};
  const float sn[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = x[2 * j], b = x[2 * j + 1];
    x[2 * j] = a * co[j] - b * sn[j];
    x[2 * j + 1] = a * sn[j] + b * co[j];
  }
}

// ------------------------------------------------- dense K rows, V^T tiles --
// One work-group per (64-key tile t, batch*head): rows 64 t .. 64 t + 63 of
// the key and value sequences ([BH][M][D], bf16 or fp32).  bf16 keys are
// turned by RoPE at their grid position (rows below T are text at (0, 0),
// row T + n is image token n) through the [P][D/4] (cos, sin) table `rope`;
// fp32 keys (pooled, already turned) are taken as they are.  Outputs:
// fp16 key rows kr[bh][row][D] (rows < M only) and the fp16 V^T tile
// vt[bh][t][d][k] = v[bh][64 t + k][d] (zero past M), each scaled by the
// tile's own power of two (kexp, vexp[bh][t]; flags[bh] set when nonzero).
template <int D, bool F32_IN>
__global__ __launch_bounds__(256) void kv_tiles_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                       const float* __restrict__ rope, u16* __restrict__ kr,
                                                       u16* __restrict__ vt, int* __restrict__ kexp,
                                                       int* __restrict__ vexp, int* __restrict__ flags, int M,
                                                       int tiles, int T, int Gw) {
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int HALF = CPR / 2;   // chunks per axis half
  constexpr int NF = D / 4;       // frequencies per axis half
  constexpr int CH = BN * CPR / 256;
  constexpr int LS = D + 8;
  __shared__ __attribute__((aligned(16))) u16 buf[BN * LS];
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int64_t bh = blockIdx.y;
  float kx[CH][8], vx[CH][8];
  float mk = 0.0f, mv = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / CPR, col = c - row * CPR;
    const int key = t * BN + row;
#pragma unroll
    for (int e = 0; e < 8; ++e) kx[i][e] = vx[i][e] = 0.0f;
    if (key < M) {
      const int64_t off = (bh * (int64_t)M + key) * D + col * 8;
      if constexpr (F32_IN) {
        const float4* kp = reinterpret_cast<const float4*>((const float*)k + off);
        const float4* vp = reinterpret_cast<const float4*>((const float*)v + off);
        const float4 k0 = kp[0], k1 = kp[1], v0 = vp[0], v1 = vp[1];
        const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kx[i][e] = kk[e];
          vx[i][e] = vv[e];
        }
      } else {
        bf8_to_f32(*reinterpret_cast<const u32x4*>((const u16*)k + off), kx[i]);
        bf8_to_f32(*reinterpret_cast<const u32x4*>((const u16*)v + off), vx[i]);
        int py = 0, px = 0;
        if (key >= T) {
          py = (key - T) / Gw;
          px = key - T - py * Gw;
        }
        // chunk col: channels 8 col .. 8 col + 7, pairs 4 (col % HALF) .. of its axis half
        rope8_f32(kx[i], reinterpret_cast<const float4*>(rope + 2 * ((col < HALF ? py : px) * NF + 4 * (col % HALF))));
      }
    }
    mk = maxabs8(kx[i], mk);
    mv = maxabs8(vx[i], mv);
  }
  const int ek = operand_exponent(block_max4(mk, red));
  const int ev = operand_exponent(block_max4(mv, red));
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / CPR, col = c - row * CPR;
    const int key = t * BN + row;
    if (key < M) *reinterpret_cast<u32x4*>(kr + (bh * (int64_t)M + key) * D + col * 8) = f16x8_scaled(kx[i], ek);
    *reinterpret_cast<u32x4*>(buf + row * LS + col * 8) = f16x8_scaled(vx[i], ev);
  }
  if (threadIdx.x == 0) {
    kexp[bh * tiles + t] = ek;
    vexp[bh * tiles + t] = ev;
    if (ek | ev) flags[bh] = 1;
  }
  __syncthreads();
  u16* dst = vt + (bh * tiles + t) * (int64_t)D * BN;
  for (int c = threadIdx.x; c < D * (BN / 8); c += 256) {
    int d = c / (BN / 8), k8 = c - d * (BN / 8);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (unsigned)buf[(8 * k8 + 2 * i) * LS + d] | ((unsigned)buf[(8 * k8 + 2 * i + 1) * LS + d] << 16);
    *reinterpret_cast<u32x4*>(dst + d * BN + 8 * k8) = o;
  }
}

// ------------------------------------------------- window work structures --
// Items workspace: counters, per-record slot / key-tile offsets, the first
// record of every base window, the (record, query tile) list and the
// (record, key tile) list of the gather.
struct ItemsWs {
  int* n_items;       // [0] attention items, [1] gather tiles
  int* slot_off;      // [max_windows] first fp32 output slot of a record
  int* kv_tile_off;   // [max_windows] first gathered key tile of a record
  int* rec_start;     // [n_base]
  int* items;         // [max_items][2]
  int* gtiles;        // [max_gtiles][2]
};

ItemsWs make_items_ws(void* ws, int max_windows, int n_base, int64_t max_items) {
  ItemsWs w;
  char* p = (char*)ws;
  w.n_items = (int*)p;
  p += align_up(2 * sizeof(int));
  w.slot_off = (int*)p;
  p += align_up(sizeof(int) * (max_windows > 0 ? max_windows : 1));
  w.kv_tile_off = (int*)p;
  p += align_up(sizeof(int) * (max_windows > 0 ? max_windows : 1));
  w.rec_start = (int*)p;
  p += align_up(sizeof(int) * (n_base > 0 ? n_base : 1));
  w.items = (int*)p;
  p += align_up(sizeof(int) * 2 * (max_items > 0 ? max_items : 1));
  w.gtiles = (int*)p;
  return w;
}

// One block: slot offsets (prefix of query areas in record order), key-tile
// offsets (prefix of ceil((kh kw + R) / 64), R the bridge and text keys a
// window can add), the first record of every base
// window, the (record, query tile) list -- whole windows first, quadrants
// after (largest key sets first) -- and the (record, key tile) list.
__global__ __launch_bounds__(256) void items_kernel(const int32_t* __restrict__ plan, ItemsWs w, int BM, int R,
                                                    int max_windows, int64_t max_items, int64_t max_gtiles) {
  __shared__ int s_item_off[4 * kMaxAxisWindows * kMaxAxisWindows];
  int nwin = plan[AREA_PH_NWIN];
  if (nwin > max_windows) nwin = max_windows;
  if (threadIdx.x == 0) {
    int it = 0;
    for (int pass = 0; pass < 2; ++pass) {
      for (int i = 0; i < nwin; ++i) {
        const int32_t* rp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * i;
        bool quad = rp[9] >= 0;
        if ((pass == 0) == quad) continue;
        s_item_off[i] = it;
        it += (rp[2] * rp[3] + BM - 1) / BM;
      }
    }
    int qs = 0, kt = 0;
    for (int i = 0; i < nwin; ++i) {
      const int32_t* rp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * i;
      w.slot_off[i] = qs;
      qs += rp[2] * rp[3];
      w.kv_tile_off[i] = kt;
      kt += (rp[6] * rp[7] + R + BN - 1) / BN;
      if (rp[9] <= 0) w.rec_start[rp[8]] = i;
    }
    w.n_items[0] = it < max_items ? it : (int)max_items;
    w.n_items[1] = kt < max_gtiles ? kt : (int)max_gtiles;
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
    int kt = (rp[6] * rp[7] + R + BN - 1) / BN;
    for (int t = threadIdx.x; t < kt; t += blockDim.x) {
      int idx = w.kv_tile_off[i] + t;
      if (idx < max_gtiles) {
        w.gtiles[2 * idx] = i;
        w.gtiles[2 * idx + 1] = t;
      }
    }
  }
}

// Bridge tokens outside each window's Halo rectangle, in ascending order:
// list[(rec * BH + bh) * R + i], count[rec * BH + bh].  One block per
// (record, batch*head).
__global__ __launch_bounds__(256) void bridge_compact_kernel(const int32_t* __restrict__ plan,
                                                             const int32_t* __restrict__ bridge, int* __restrict__ list,
                                                             int* __restrict__ count, int R, int Gw, int64_t BH) {
  __shared__ int s_wave[4];
  const int rec = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (rec >= plan[AREA_PH_NWIN]) return;
  const int32_t* rp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * rec;
  const int ky0 = rp[4], kx0 = rp[5], kh = rp[6], kw = rp[7];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int* dst = list + ((int64_t)rec * BH + bh) * R;
  int base = 0;
  for (int j0 = 0; j0 < R; j0 += 256) {
    int j = j0 + threadIdx.x;
    int tok = 0;
    bool keep = false;
    if (j < R) {
      tok = bridge[bh * R + j];
      int y = tok / Gw, x = tok - y * Gw;
      keep = !(y >= ky0 && y < ky0 + kh && x >= kx0 && x < kx0 + kw);
    }
    uint64_t m = __ballot(keep);
    int before = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
    if (lane == 0) s_wave[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int i = 0; i < wave; ++i) off += s_wave[i];
    if (keep) dst[off + before] = tok;
    int tot = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    __syncthreads();
    base += tot;
  }
  if (threadIdx.x == 0) count[(int64_t)rec * BH + bh] = base;
}

// Gathers one 64-key tile of a window's key set: slot s < kh*kw is the Halo
// rectangle token s (row-major), then the compacted outside bridge tokens,
// then the T text tokens, then zero rows.  Sequences hold the T text rows
// first, image token n at row T + n.  K rows are turned by RoPE at their
// token's grid position (text rows at (0, 0), unturned) through the (cos,
// sin) table `rope`; V rows are written transposed.  Both are fp16, scaled by
// the tile's own power of two (kexp, vexp[bh][tile]; flags[bh] set when
// nonzero), as kv_tiles_kernel does for dense key sets.
template <int D>
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ plan, const int* __restrict__ gtiles,
                                                     const int* __restrict__ n_items, const int* __restrict__ kv_tile_off,
                                                     const int* __restrict__ list, const int* __restrict__ count,
                                                     const u16* __restrict__ k, const u16* __restrict__ v,
                                                     const float* __restrict__ rope, u16* __restrict__ kg,
                                                     u16* __restrict__ vg, int* __restrict__ kexp, int* __restrict__ vexp,
                                                     int* __restrict__ flags, int64_t cap_tiles, int R, int Tt, int Gw,
                                                     int N, int64_t BH) {
  constexpr int CPR = D / 8;
  constexpr int HALF = CPR / 2;  // chunks per axis half
  constexpr int NF = D / 4;      // frequencies per axis half
  constexpr int CH = BN * CPR / 256;
  constexpr int LS = D + 8;
  __shared__ __attribute__((aligned(16))) u16 buf[BN * LS];
  __shared__ int s_tok[BN];
  __shared__ int s_py[BN], s_px[BN];
  __shared__ float red[4];
  const int g = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (g >= n_items[1]) return;
  const int rec = gtiles[2 * g], t = gtiles[2 * g + 1];
  const int32_t* rp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * rec;
  const int ky0 = rp[4], kx0 = rp[5], kw = rp[7];
  const int nrect = rp[6] * kw;
  const int cnt = R > 0 ? count[(int64_t)rec * BH + bh] : 0;
  const int gt = kv_tile_off[rec] + t;  // the tile's index among the gathered tiles
  if (threadIdx.x < BN) {
    int s = t * BN + threadIdx.x;
    int row = -1;  // sequence row of the slot's token
    int py = 0, px = 0;  // its grid position (text: (0, 0))
    if (s < nrect) {
      int yy = s / kw;
      py = ky0 + yy;
      px = kx0 + (s - yy * kw);
      row = Tt + py * Gw + px;
    } else if (s - nrect < cnt) {
      const int tok = list[((int64_t)rec * BH + bh) * R + (s - nrect)];
      py = tok / Gw;
      px = tok - py * Gw;
      row = Tt + tok;
    } else if (s - nrect - cnt < Tt) {
      row = s - nrect - cnt;
    }
    s_tok[threadIdx.x] = row;
    s_py[threadIdx.x] = py;
    s_px[threadIdx.x] = px;
  }
  __syncthreads();
  const u16* ksrc = k + bh * (int64_t)(Tt + N) * D;
  const u16* vsrc = v + bh * (int64_t)(Tt + N) * D;
  u16* kdst = kg + (bh * cap_tiles + gt) * (int64_t)BN * D;
  float kx[CH][8], vx[CH][8];
  float mk = 0.0f, mv = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / CPR, col = c - row * CPR;
    const int tok = s_tok[row];
#pragma unroll
    for (int e = 0; e < 8; ++e) kx[i][e] = vx[i][e] = 0.0f;
    if (tok >= 0) {
      // chunk col: channels 8 col .. 8 col + 7, rotation pairs 4 (col % HALF) ..
      // of the row (first half) or column (second half) axis
      const int pos = col < HALF ? s_py[row] : s_px[row];
      bf8_to_f32(*reinterpret_cast<const u32x4*>(ksrc + (int64_t)tok * D + col * 8), kx[i]);
      bf8_to_f32(*reinterpret_cast<const u32x4*>(vsrc + (int64_t)tok * D + col * 8), vx[i]);
      rope8_f32(kx[i], reinterpret_cast<const float4*>(rope + 2 * (pos * NF + 4 * (col % HALF))));
    }
    mk = maxabs8(kx[i], mk);
    mv = maxabs8(vx[i], mv);
  }
  const int ek = operand_exponent(block_max4(mk, red));
  const int ev = operand_exponent(block_max4(mv, red));
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / CPR, col = c - row * CPR;
    *reinterpret_cast<u32x4*>(kdst + row * D + col * 8) = f16x8_scaled(kx[i], ek);
    *reinterpret_cast<u32x4*>(buf + row * LS + col * 8) = f16x8_scaled(vx[i], ev);
  }
  if (threadIdx.x == 0) {
    kexp[bh * cap_tiles + gt] = ek;
    vexp[bh * cap_tiles + gt] = ev;
    if (ek | ev) flags[bh] = 1;
  }
  __syncthreads();
  u16* vdst = vg + (bh * cap_tiles + gt) * (int64_t)D * BN;
  for (int c = threadIdx.x; c < D * (BN / 8); c += 256) {
    int d = c / (BN / 8), k8 = c - d * (BN / 8);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (unsigned)buf[(8 * k8 + 2 * i) * LS + d] | ((unsigned)buf[(8 * k8 + 2 * i + 1) * LS + d] << 16);
    *reinterpret_cast<u32x4*>(vdst + d * BN + 8 * k8) = o;
  }
}

// -------------------------------------------------------------- attention --
struct AttnArgs {
  const u16* q;        // un-rotated queries, bf16 [BH][q_rows][D]
  const float4* rope;  // [D/8][rope_P] (cos, sin) of frequencies 2i, 2i+1 at axis position p
  int rope_P;          // positions per frequency pair (max(Gh, Gw))
  int q_text;          // rows below q_text are text (not rotated); row q_text + n is image token n
  const u16* k;        // fp16 key rows [BH][k_rows][D]
  const u16* vt;       // fp16 V^T tiles [BH][k_tiles][D][64]
  u16* out;            // bf16 [BH][q_rows][D]
  int64_t BH;
  int Nq;              // dense mode: queries per head, rows q0 .. q0 + Nq - 1
  int q0, q_rows;      // first query row (window mode: image token n is row q0 + n); rows per head
  int64_t k_rows, k_tiles;  // per-(batch*head) strides of k and vt
  const int* kexp;     // [BH][k_tiles] power-of-two exponent of each key tile (stored K * 2^-e)
  const int* vexp;     // [BH][k_tiles] the same for the V^T tiles
  const int* flags;    // [BH] nonzero: some tile of the (batch, head) has a nonzero exponent
  int* redo;           // [0]: count, then the logical ids of the items the scaled kernel runs
  int* ctr;            // [8] per-XCD work counters of the persistent plain kernel
  int n_kv;            // dense mode: keys per query
  int n_qtiles;        // dense mode: query tiles per head
  float c;             // log2(e) / sqrt(D)
  // window mode
  const int32_t* plan;
  const int32_t* wsum;
  const int* items;        // [max_items][2] = (record, query tile)
  const int* n_items;
  const int* slot_off;     // per record: first fp32 output slot
  const int* kv_tile_off;  // per record: first gathered key tile
  const int* bcount;       // [record][BH] bridge tokens kept
  float* slots;            // [slot][BH][D] fp32 outputs of overlapped tokens
  int Gw;              // grid width (query positions)
  int R, T;            // window mode: bridge slots and text keys ending every key set
  int64_t max_items;
};

// LDS tile layouts (one stage = one 64-key tile).  Rows are unpadded so that
// a tile can be filled by global->LDS DMA (each lane of a wave writes 16
// bytes at base + 16 * lane); bank conflicts are avoided by XOR-swizzling the
// 16-byte chunk index with the row index instead:
//  * K: row r (D*2 bytes) holds key perm(r) (bits 2 and 3 of r swapped, the
//    MFMA row order of the score tile); logical chunk c sits at c ^ swz(r).
//  * V^T: row d (64 keys, 128 bytes) of the transposed tile; logical chunk c
//    (8 keys) sits at c ^ swz(d).
// swz() makes the 8 (or 16) lanes served together by a 128-bit read hit
// distinct banks under both the 32-bank and the 64-bank arrangement.
template <int ROW_BYTES>
__device__ __attribute__((always_inline)) inline int swz(int r) {
  if constexpr (ROW_BYTES >= 256) return r & 15;
  else return (r & 7) ^ ((r >> 3) & 1);
}

__device__ __attribute__((always_inline)) inline int key_perm(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// LDS element offset of phase A's K fragment j (block kb = j & 1 of 32
// keys, 16-channel step j >> 1).
template <int D>
__device__ __attribute__((always_inline)) inline int k_frag_off(int j, int n, int hi) {
  const int kd = j >> 1, kb = j & 1;
  return (32 * kb + n) * D + (((2 * kd + hi) ^ swz<D * 2>(n)) * 8);
}

// LDS element offset of phase B's V^T fragment j (block db = j % (D/32) of
// 32 d-rows, 16-key step j / (D/32)).
template <int D>
__device__ __attribute__((always_inline)) inline int vt_frag_off(int j, int n, int hi) {
  constexpr int DB = D / 32;
  const int ks = j / DB, db = j % DB;
  return (32 * db + n) * BN + (((2 * ks + hi) ^ swz<BN * 2>(n)) * 8);
}

typedef __attribute__((address_space(3))) void* lptr_t;

// Work-group of the attention kernel: kAttnWaves waves of 32 kAttnQG queries.
constexpr int kThreads = 64 * kAttnWaves;

// DMA of one tile's K rows (issue_k) or V^T rows (issue_v) into an LDS
// stage, CH 16-byte chunks per thread, with buffer loads: a per-tile buffer
// resource (scalar base and byte count) plus a loop-invariant lane offset.
// K rows past the last key of the set fall outside the resource's range and
// read as zero (their scores are masked).  `wave` is wave-uniform, so the LDS
// addresses (M0) are scalar.
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format

template <int D>
__device__ __attribute__((always_inline)) inline void issue_k(u16* ks, int tile, int tid, int wave, int nkv,
                                                              const u16* kbase) {
  constexpr int KCH = D / 8;  // 16-byte chunks per K row
  constexpr int CH = BN * D / 8 / kThreads;
  const int rows = __builtin_amdgcn_readfirstlane(min(max(nkv - tile * BN, 0), BN));
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)tile * BN * D), (short)0, rows * D * 2, kBufferWord3);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int p = i * kThreads + tid;  // LDS chunk written by this lane
    const int r = p / KCH, pc = p - r * KCH;
    const int c = pc ^ swz<D * 2>(r);
    const unsigned off = (unsigned)(key_perm(r) * (D * 2) + c * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(ks + (i * kThreads + wave * 64) * 8), 16, off, 0, 0, 0);
  }
}

template <int D>
__device__ __attribute__((always_inline)) inline void issue_v(u16* vt, int tile, int tid, int wave,
                                                              const u16* vtbase) {
  constexpr int VCH = BN / 8;  // 16-byte chunks per V^T row
  constexpr int CH = BN * D / 8 / kThreads;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vtbase + (int64_t)tile * D * BN), (short)0, D * BN * 2, kBufferWord3);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int p = i * kThreads + tid;
    const int d = p / VCH, pc = p - d * VCH;
    const int c = pc ^ swz<BN * 2>(d);
    const unsigned off = (unsigned)(d * (BN * 2) + c * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(vt + (i * kThreads + wave * 64) * 8), 16, off, 0, 0, 0);
  }
}

// S^T (keys x queries) of one tile for the wave's QG groups of 32 queries.
// MFMA row n of block kb reads LDS row 32 kb + n, which holds key
// perm(32 kb + n).
template <int D, int QG>
__device__ __attribute__((always_inline)) inline void tile_scores(f32x16 (&s)[QG][2], const u16* ks, int n, int hi,
                                                                  const f16x8 (&qf)[QG][D / 16]) {
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[g][kb][i] = 0.0f;
  const int sw = swz<D * 2>(n);
#pragma unroll
  for (int kd = 0; kd < D / 16; ++kd) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u16* kr = ks + (32 * kb + n) * D + (((2 * kd + hi) ^ sw) * 8);
      f16x8 af = *reinterpret_cast<const f16x8*>(kr);
#pragma unroll
      for (int g = 0; g < QG; ++g) s[g][kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, qf[g][kd], s[g][kb], 0, 0, 0);
    }
  }
}

// Keys at or beyond `valid` (tail of the last tile) get a -inf score.  S^T
// register 8*jj + i of block kb is key 32 kb + 16 jj + 8 hi + i.
template <int QG>
__device__ __attribute__((always_inline)) inline void mask_tail(f32x16 (&s)[QG][2], int valid, int hi) {
  const int lim = valid - 8 * hi;
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[g][kb][i] = 32 * kb + 16 * (i >> 3) + (i & 7) < lim ? s[g][kb][i] : -INFINITY;
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

// Operand fragments are read from LDS kFragAhead MFMAs before their use.
// Each MFMA of phase A is paired with the softmax work of two scores: two
// exp2 (transcendental unit), then the pair's fp16 conversion and its dot2
// into the P sum, in groups of up to kValuA VALU instructions.  Phase B's
// MFMAs carry no softmax work.
constexpr int kFragAhead = 3;
constexpr int kTransA = 2;
constexpr int kValuA = 3;

// sched_group_barrier masks (VALU excludes the transcendental instructions,
// which have their own class)
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedTrans = 0x400;

__device__ __attribute__((always_inline)) inline const u16* uniform_ptr(const u16* p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (const u16*)(((unsigned long long)hi << 32) | lo);
}

__device__ __attribute__((always_inline)) inline f16x8 lds_frag(const u16* stage, int elem_off) {
  return *reinterpret_cast<const f16x8*>(stage + elem_off);
}

// Phase A of one step: S^T of the next tile for the wave's QG query groups
// (2 D/16 K fragments, each read once from LDS and used by every group)
// while the VALU turns the current scores into fp16 P^T = exp2(scores) and
// sums each lane's P (psum).
// The caller has read the first kFragAhead K fragments (fr); the reads that
// would run past the last K fragment fetch phase B's first V^T fragments
// (vfr) instead, so phase B starts without waiting for LDS.
// Scores are in log2 units relative to the running maximum m: the queries
// carry log2(e)/sqrt(D), and the first MFMA of each accumulator starts from
// nm = -m instead of zero, so no per-score scale or subtraction is left.
// With ZERO_START (the scaled loop) the accumulators start from zero and the
// caller shifts and rescales the raw scores itself.  With LAST (an item's
// last tile) no MFMA runs: only P and its sums, and phase B's first V^T
// fragments are read.
template <int D, int QG, bool ZERO_START = false, bool LAST = false>
__device__ __attribute__((always_inline)) inline void phase_a(f32x16 (&sn)[QG][2], const u16* ks, int n, int hi,
                                                              const f16x8 (&qf)[QG][D / 16],
                                                              const f32x16 (&sc)[QG][2], const f32x16 (&nm)[QG],
                                                              f16x8 (&pf)[QG][4], f16x8 (&fr)[kFragAhead],
                                                              const u16* vt, f16x8 (&vfr)[kFragAhead],
                                                              float (&psum)[QG]) {
  constexpr int NT = 2 * (D / 16);
  constexpr int EPM = 32 * QG / NT;  // scores turned into P per fragment
  constexpr int PF = kFragAhead;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 ph[QG][16];
  const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
  float ps[QG][2];
#pragma unroll
  for (int g = 0; g < QG; ++g) ps[g][0] = ps[g][1] = 0.0f;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if constexpr (LAST) {
      if (j < PF) vfr[j] = lds_frag(vt, vt_frag_off<D>(j, n, hi));
    } else {
      const f16x8 f = fr[j % PF];
      if (j + PF < NT) fr[j % PF] = lds_frag(ks, k_frag_off<D>(j + PF, n, hi));
      else vfr[j + PF - NT] = lds_frag(vt, vt_frag_off<D>(j + PF - NT, n, hi));
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        if constexpr (ZERO_START) {
          const f32x16 zero = {};
          sn[g][j & 1] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(f, qf[g][j >> 1], j < 2 ? zero : sn[g][j & 1], 0, 0, 0);
        } else {
          sn[g][j & 1] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(f, qf[g][j >> 1], j < 2 ? nm[g] : sn[g][j & 1], 0, 0, 0);
        }
      }
    }
    // P of EPM scores, converted in pairs (one packed conversion per pair)
#pragma unroll
    for (int e = EPM * j; e < EPM * j + EPM; e += 2) {
      const int g = e >> 5, x = e & 31;
      const f32x2 p2 = {__builtin_amdgcn_exp2f(sc[g][x >> 4][x & 15]),
                        __builtin_amdgcn_exp2f(sc[g][(x + 1) >> 4][(x + 1) & 15])};
      ph[g][x >> 1] = __builtin_convertvector(p2, f16x2);
      ps[g][(x >> 1) & 1] = __builtin_amdgcn_fdot2(ph[g][x >> 1], one2, ps[g][(x >> 1) & 1], false);
    }
  }
#pragma unroll
  for (int g = 0; g < QG; ++g) psum[g] = ps[g][0] + ps[g][1];
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[g][r][2 * i] = ph[g][4 * r + i][0];
        pf[g][r][2 * i + 1] = ph[g][4 * r + i][1];
      }
  // issue order: per fragment its MFMAs, the next read (K, then V^T for
  // phase B), the exp2 of EPM scores and the conversion of the previous pair
  if constexpr (LAST) return;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, QG, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedTrans, kTransA * EPM / 2, 0);
    if (j > 0) __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuA * EPM / 2, 0);
  }
}

// Phase B of one step: O^T += V^T P^T for every group (4 D/32 V^T
// fragments, each read once; the first kFragAhead already in fr).
template <int D, int QG>
__device__ __attribute__((always_inline)) inline void phase_b(f32x16 (&o)[QG][D / 32], const u16* vt, int n, int hi,
                                                              const f16x8 (&pf)[QG][4], f16x8 (&fr)[kFragAhead]) {
  constexpr int DB = D / 32;
  constexpr int NT = 4 * DB;
  constexpr int PF = kFragAhead;

#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const f16x8 f = fr[j % PF];
    if (j + PF < NT) fr[j % PF] = lds_frag(vt, vt_frag_off<D>(j + PF, n, hi));
#pragma unroll
    for (int g = 0; g < QG; ++g)
      o[g][j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f, pf[g][j / DB], o[g][j % DB], 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, QG, 0);
    if (j + PF < NT) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
}

// Work-groups per CU the register budget is sized for: two four-wave groups,
// else one.
constexpr int kAttnGroupsPerCu = kAttnQG == 1 && kAttnWaves == 4 ? 2 : 1;

// A work item: 256 queries of one (batch, head) -- a query tile of the dense
// sequence, or of one window record -- over the item's whole key set.  The
// fields are wave-uniform.
struct Item {
  bool valid;
  int L, bh, qtile, rec, qy0, qx0, qh, qw, nq, nkv;
  int64_t t0;                // first key tile of the item's key set
  const u16* kbase;
  const u16* vtbase;
  const u16* qbase;
};

template <int D, bool WIN>
__device__ __attribute__((always_inline)) inline Item decode_item(const AttnArgs& a, int L) {
  Item it;
  it.valid = false;
  it.L = L;
  it.bh = it.qtile = it.rec = it.qy0 = it.qx0 = it.qh = it.nq = it.nkv = 0;
  it.qw = 1;
  it.t0 = 0;
  it.kbase = it.vtbase = it.qbase = nullptr;
  if (L < 0) return it;
  int64_t bh;
  if constexpr (WIN) {
    const int ni = a.n_items[0];  // items per (batch, head)
    if (ni <= 0) return it;
    bh = L / ni;
    const int64_t k = L - bh * ni;
    if (bh >= a.BH) return it;
    it.rec = a.items[2 * k];
    it.qtile = a.items[2 * k + 1];
    const int32_t* rp = a.plan + AREA_PLAN_HEADER + AREA_PLAN_REC * it.rec;
    it.qy0 = rp[0];
    it.qx0 = rp[1];
    it.qh = rp[2];
    it.qw = rp[3];
    it.nq = it.qh * it.qw;
    it.nkv = rp[6] * rp[7] + (a.R > 0 ? a.bcount[(int64_t)it.rec * a.BH + bh] : 0) + a.T;
    it.t0 = a.kv_tile_off[it.rec];
  } else {
    bh = L / a.n_qtiles;
    it.qtile = (int)(L - bh * a.n_qtiles);
    if (bh >= a.BH) return it;
    it.nq = a.Nq;
    it.nkv = a.n_kv;
  }
  it.bh = (int)bh;
  // the buffer resources of the tile DMAs need wave-uniform bases and sizes
  it.nkv = __builtin_amdgcn_readfirstlane(it.nkv);
  it.kbase = uniform_ptr(a.k + bh * a.k_rows * D + it.t0 * BN * D);
  it.vtbase = uniform_ptr(a.vt + (bh * a.k_tiles + it.t0) * (int64_t)D * BN);
  it.qbase = a.q + (bh * (int64_t)a.q_rows + a.q0) * D;
  it.valid = true;
  return it;
}

// The lane's queries of an item: token rows, validity, and the raw bf16
// chunks with their (cos, sin), loaded ahead of the rotation so that the load
// latency overlaps the first tile DMAs (or the previous item's epilogue).
template <int D>
struct Queries {
  int qtok[kAttnQG];
  bool qvalid[kAttnQG];
  u32x4 qraw[kAttnQG][D / 16];
  float4 qcs[kAttnQG][D / 16][2];
};

// The lane's query token rows in the item and their validity.  Each call
// rebuilds them from the item, so that nothing lane-derived has to survive
// the key loop.
template <bool WIN>
__device__ __attribute__((always_inline)) inline void query_tokens(const AttnArgs& a, const Item& it,
                                                                   int (&qtok)[kAttnQG], bool (&qvalid)[kAttnQG]) {
  constexpr int QG = kAttnQG, BM = kAttnBM;
  const int tid = (int)threadIdx.x;
  const int n = tid & 31, wave = tid >> 6;
  // the grid width behind an empty asm: its division reciprocal is formed
  // per item, not held across the key loop
  int gw = a.Gw;
  asm volatile("" : "+s"(gw));
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int t = it.qtile * BM + wave * 32 * QG + 32 * g + n;
    qvalid[g] = t < it.nq;
    if constexpr (WIN) {
      const int yy = qvalid[g] ? t / it.qw : 0;
      const int xx = qvalid[g] ? t - yy * it.qw : 0;
      qtok[g] = (it.qy0 + yy) * gw + it.qx0 + xx;
    } else {
      qtok[g] = qvalid[g] ? t : 0;
    }
  }
}

template <int D, bool WIN>
__device__ __attribute__((always_inline)) inline void load_queries(const AttnArgs& a, const Item& it,
                                                                   Queries<D>& q) {
  constexpr int QG = kAttnQG, KD = D / 16;
  const int tid = (int)threadIdx.x;
  const int hi = (tid & 63) >> 5;
  int gw = a.Gw;
  asm volatile("" : "+s"(gw));
  query_tokens<WIN>(a, it, q.qtok, q.qvalid);
  // MFMA B operand: chunk 2 kd + hi (channels 16 kd + 8 hi ..) of the
  // lane's query, turned by RoPE at its grid position (chunks of the first
  // half follow the row, the others the column; text rows sit at (0, 0)).
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int64_t row = (int64_t)a.q0 + q.qtok[g];
    int py = 0, px = 0;
    if (row >= a.q_text) {
      const int img = (int)(row - a.q_text);
      py = img / gw;
      px = img - py * gw;
    }
    const u32x4* qrow = reinterpret_cast<const u32x4*>(it.qbase + (int64_t)q.qtok[g] * D);
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const int ch = 2 * kd + hi;
      const int pos = kd < KD / 2 ? py : px;
      // frequencies 4 (ch % KD) .. + 3: pairs 2 (ch % KD) and 2 (ch % KD) + 1
      const float4* cs = a.rope + (int64_t)(2 * (ch % KD)) * a.rope_P + pos;
      q.qraw[g][kd] = qrow[ch];
      q.qcs[g][kd][0] = cs[0];
      q.qcs[g][kd][1] = cs[a.rope_P];
    }
  }
}

// DMAs of an item's first tiles: K tile 0 and V^T tile 0 into stage 0, K
// tile 1 (or 0 again) into stage 1.
template <int D>
__device__ __attribute__((always_inline)) inline void issue_first(const Item& it, u16* ks0, u16* vt0, u16* ks1) {
  const int tid = (int)threadIdx.x;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = (it.nkv + BN - 1) / BN;
  issue_k<D>(ks0, 0, tid, wave_u, it.nkv, it.kbase);
  issue_v<D>(vt0, 0, tid, wave_u, it.vtbase);
  issue_k<D>(ks1, min(1, nt - 1), tid, wave_u, it.nkv, it.kbase);
}

// Claims the next work item from the per-XCD counters ctr[8]: logical ids
// x * per .. x * per + per - 1 (those below total) belong to XCD x; an XCD
// whose share is spent takes from the others in turn.  raw is the value this
// work-group already drew from its own XCD's counter.  -1 when every share is
// spent.
__device__ inline int claim_from(int* ctr, int xcd, int per, int64_t total, int raw) {
  if (raw < per && (int64_t)xcd * per + raw < total) return xcd * per + raw;
  for (int k = 1; k < 8; ++k) {
    const int x = (xcd + k) & 7;
    const int i = atomicAdd(&ctr[x], 1);
    if (i < per && (int64_t)x * per + i < total) return x * per + i;
  }
  return -1;
}

// Everything of an item between its query loads and its epilogue: rotation
// of the queries (with their exponents), then, unless the item needs the
// scaled loop (the plain kernel lists it and returns true), the first tile's
// scores and the software-pipelined loop over the key tiles.  The plain
// kernel also resolves the next item here: `fut` (thread 0's draw from its
// XCD's counter) becomes `look`.  s_sync: kAttnWaves + 1 LDS words (the
// waves' votes, then the next item's id).
template <int D, bool WIN, bool SCALED>
__device__ __attribute__((always_inline)) inline bool compute_item(
    const AttnArgs& a, const Item& it, Queries<D>& qs, u16* ks0, u16* vt0, u16* ks1, u16* vt1,
    f32x16 (&o)[kAttnQG][D / 32], float (&l_run)[kAttnQG], int& ev_cur, int* s_sync, int* ctr, int xcd, int per,
    int64_t total, int fut, int& look) {
  constexpr int QG = kAttnQG;
  constexpr int KD = D / 16;
  constexpr int DB = D / 32;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hi = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int bh = it.bh;
  const int64_t t0 = it.t0;
  const int nkv = it.nkv;
  const u16* kbase = it.kbase;
  const u16* vtbase = it.vtbase;
  const int nt = (nkv + BN - 1) / BN;
  const float c = a.c;

  f16x8 qf[QG][KD];
  int eq[QG];         // per query row: operands carry q * log2(e)/sqrt(D) * 2^-eq
  float lsc = 1.0f;   // 2^-d of the tile whose P is turned next (scaled loop)
  f32x16 nm[QG];      // -m, the running maximum (log2 units), in all 16 registers
  ev_cur = 0;         // V^T unit: O holds O_true * 2^-ev_cur (scaled loop)
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    l_run[g] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[g][db][i] = 0.0f;
  }

  // Software pipeline over key tiles: while the matrix cores compute the
  // scores of tile j+1, the VALU turns the scores of tile j into P and sums
  // it; then they compute O += P V for tile j.  A P sum that flags a larger
  // score moves the maximum between the two phases (rare).  K tile j+1 and
  // V tile j are resident during step j; K tile
  // j+2 and V tile j+1 stream into the other stages meanwhile.
  // The scaled variant (SC) handles nonzero exponents: its score
  // accumulators start from zero, so a tile's raw scores are
  // s * 2^-(eq + ek); after phase B they are moved to s - m in fp32 for the
  // next step.  A V^T tile stored at 2^-ev adds ev - ev_cur to its scores
  // (P carries 2^(ev - ev_cur)), and a tile with ev above ev_cur first moves
  // O to the new unit, so P never grows; l stays in true units.
  // The item's last step (last_tag) reads no K fragments, starts no DMA and
  // computes no scores: phase A only turns the current scores into P.
  auto step = [&](auto scaled_tag, auto last_tag, f32x16 (&scur)[QG][2], f32x16 (&snext)[QG][2], const u16* ksn,
                  const u16* vtc, int j, u16* kdma, int ktile, u16* vdma, int vtile)
      __attribute__((always_inline)) {
    constexpr bool SC = decltype(scaled_tag)::value;
    constexpr bool LT = decltype(last_tag)::value;
    f16x8 kfr[kFragAhead];
    if constexpr (!LT) {
      // phase A's first K fragments, read ahead of the tile DMAs so their
      // LDS latency overlaps them
#pragma unroll
      for (int jj = 0; jj < kFragAhead; ++jj)
        kfr[jj] = lds_frag(ksn, k_frag_off<D>(jj, n, hi));
      __builtin_amdgcn_sched_barrier(0);
      // DMAs of the next tiles into the two free stages
      issue_k<D>(kdma, ktile, tid, wave_u, nkv, kbase);
      issue_v<D>(vdma, vtile, tid, wave_u, vtbase);
    }
    f16x8 pf[QG][4];
    f16x8 vfr[kFragAhead];
    float psum[QG];
    phase_a<D, QG, SC, LT>(snext, ksn, n, hi, qf, scur, nm, pf, kfr, vtc, vfr, psum);
    // keep P's computation in this block: its only use is after the branch
#pragma unroll
    for (int g = 0; g < QG; ++g)
      asm volatile("" : "+v"(pf[g][0]), "+v"(pf[g][1]), "+v"(pf[g][2]), "+v"(pf[g][3]), "+v"(psum[g]));
    // Lazy maximum: the scores were taken relative to the running maximum m,
    // so P <= 1 unless the tile holds a larger score.  Each lane's P sum
    // bounds every P it holds; while it stays at most 2^8, P fits fp16 with
    // room to spare and m stays.  Otherwise (rare) m moves to the tile's
    // maximum: O and l are rescaled, P is recomputed, and the next tile's
    // scores and the accumulator start are shifted to the new m.
    bool big = false;
#pragma unroll
    for (int g = 0; g < QG; ++g) big |= !(psum[g] <= kPsumMax);
    if (__any(big)) {
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        float m = fmaxf(scur[g][0][0], scur[g][0][1]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) m = fmaxf(m, scur[g][kb][i]);
        const float mt = pair_max(m);
        const float dlt = mt > 0.0f ? mt : 0.0f;
        const float alpha = __builtin_amdgcn_exp2f(-dlt);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[g][db][i] *= alpha;
        l_run[g] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          nm[g][i] -= dlt;
          if constexpr (!SC) {  // raw scores of the scaled loop take the new m at their fix-up
            snext[g][0][i] -= dlt;
            snext[g][1][i] -= dlt;
          }
        }
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
        float s0 = 0.0f;
#pragma unroll
        for (int x = 0; x < 32; x += 2) {
          const f16x2 p2 = {(_Float16)__builtin_amdgcn_exp2f(scur[g][x >> 4][x & 15] - dlt),
                            (_Float16)__builtin_amdgcn_exp2f(scur[g][(x + 1) >> 4][(x + 1) & 15] - dlt)};
          pf[g][x >> 3][x & 7] = p2[0];
          pf[g][x >> 3][(x & 7) + 1] = p2[1];
          s0 = __builtin_amdgcn_fdot2(p2, one2, s0, false);
        }
        psum[g] = s0;
      }
    }
    const int valid = nkv - (j + 1) * BN;
    if constexpr (!LT) {
      if (valid < BN) mask_tail<QG>(snext, valid, hi);
    }
    phase_b<D, QG>(o, vtc, n, hi, pf, vfr);
    if constexpr (SC) {
#pragma unroll
      for (int g = 0; g < QG; ++g) l_run[g] += psum[g] * lsc;
      if (j + 1 < nt) {
        const int64_t eb = bh * a.k_tiles + t0 + j + 1;
        const int ek = a.kexp[eb], ev = a.vexp[eb];
        int d = ev - ev_cur;
        if (d > 0) {
          const float al = ldexpf(1.0f, -d);
#pragma unroll
          for (int g = 0; g < QG; ++g)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
              for (int i = 0; i < 16; ++i) o[g][db][i] *= al;
          ev_cur = ev;
          d = 0;
        }
        lsc = ldexpf(1.0f, -d);
#pragma unroll
        for (int g = 0; g < QG; ++g) {
          const float sc = ldexpf(1.0f, eq[g] + ek);
          const float cc = nm[g][0] + (float)d;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) snext[g][kb][i] = fmaf(snext[g][kb][i], sc, cc);
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < QG; ++g) l_run[g] += psum[g];
    }
  };

  // Stage use: K tile t in ks[t % 2], V tile t in vt[t % 2].  Each step
  // reads its first K fragments, starts the DMAs into the two free stages,
  // computes, then waits for its own DMAs and syncs; every step ends with
  // one barrier, so an item takes nt of them.  No DMA is outstanding at a
  // branch merge.  The item's first three tile DMAs are already in flight.
  f32x16 sa[QG][2], sb[QG][2];
  // Each query row carries its own power-of-two exponent eq (operand_exponent
  // of the row's largest turned and scaled magnitude, the two lanes of a
  // query column agreeing); a row with eq != 0 is converted again at
  // 2^-eq.
  bool any_eq = false;
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    float mx = 0.0f;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
      qf[g][kd] =
          __builtin_bit_cast(f16x8, rope8_f16_max(qs.qraw[g][kd], qs.qcs[g][kd][0], qs.qcs[g][kd][1], c, mx));
    eq[g] = operand_exponent(pair_max(qs.qvalid[g] ? mx : 0.0f));
    if (eq[g] != 0) {
      any_eq = true;
#pragma unroll
      for (int kd = 0; kd < KD; ++kd)
        qf[g][kd] = __builtin_bit_cast(
            f16x8, rope8_f16_max(qs.qraw[g][kd], qs.qcs[g][kd][0], qs.qcs[g][kd][1], c, mx, eq[g]));
    }
  }
  // An item runs the scaled loop when a query row or a key or value tile of
  // its (batch, head) carries a nonzero exponent; the plain kernel lists
  // such an item for the scaled kernel and moves on once its DMAs have
  // landed.  The same barrier publishes the next item's id.
  constexpr bool scaled = SCALED;
  if constexpr (!SCALED) {
    // a work-group vote: each wave posts whether any of its rows has an
    // exponent (every wave writes its word, so none needs clearing)
    const bool wave_eq = __ballot(any_eq ? 1 : 0) != 0;
    if (lane == 0) s_sync[wave] = wave_eq ? 1 : 0;
    if (tid == 0) s_sync[kAttnWaves] = claim_from(ctr, xcd, per, total, fut);
    __syncthreads();
    int votes = 0;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) votes |= s_sync[w];
    const bool hand_off = votes != 0 || a.flags[bh] != 0;
    look = __builtin_amdgcn_readfirstlane(s_sync[kAttnWaves]);
    if (hand_off) {
      if (tid == 0) a.redo[1 + atomicAdd(a.redo, 1)] = it.L;
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();  // every wave has read s_sync before it is written again
      return true;
    }
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  if constexpr (scaled) {
    tile_scores<D, QG>(sa, ks0, n, hi, qf);
    // raw scores are s * 2^-(eq + ek); the first tile also fixes the V unit
    const int64_t eb = (int64_t)bh * a.k_tiles + t0;
    const int ek0 = a.kexp[eb];
    ev_cur = a.vexp[eb];
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      const float sc = ldexpf(1.0f, eq[g] + ek0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sa[g][kb][i] *= sc;
    }
  } else {
    tile_scores<D, QG>(sa, ks0, n, hi, qf);
  }
  if (nkv < BN) mask_tail<QG>(sa, nkv, hi);
  // the first tile sets the running maximum (every query has a key there)
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    float mx = fmaxf(sa[g][0][0], sa[g][0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sa[g][kb][i]);
    const float m0 = pair_max(mx);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sa[g][0][i] -= m0;
      sa[g][1][i] -= m0;
      nm[g][i] = -m0;
    }
  }
  __syncthreads();
  bool any_q = false;
#pragma unroll
  for (int g = 0; g < QG; ++g) any_q |= qs.qvalid[g];
  if (__any(any_q)) {
    // Paired steps while at least three tiles remain, then one or two
    // steps: the last one turns the last tile's scores into P and adds
    // P V only, with no scores and no DMA past the end.  With two tiles
    // left, the next-to-last step's scores move into sa first, so that one
    // copy of the last step serves both parities; that step's K DMA
    // reloads the last K tile (unused), as the idle waves' mirror does.
    auto walk = [&](auto scaled_tag) __attribute__((always_inline)) {
      int j = 0;
      for (; j + 2 < nt; j += 2) {
        step(scaled_tag, std::false_type{}, sa, sb, ks1, vt0, j, ks0, j + 2, vt1, j + 1);
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        __syncthreads();
        step(scaled_tag, std::false_type{}, sb, sa, ks0, vt1, j + 1, ks1, min(j + 3, nt - 1), vt0, j + 2);
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        __syncthreads();
      }
      const u16* vt_last = vt0;
      if (j + 2 == nt) {
        step(scaled_tag, std::false_type{}, sa, sb, ks1, vt0, j, ks0, j + 1, vt1, j + 1);
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        __syncthreads();
#pragma unroll
        for (int g = 0; g < QG; ++g) {
          sa[g][0] = sb[g][0];
          sa[g][1] = sb[g][1];
        }
        vt_last = vt1;
        ++j;
      }
      step(scaled_tag, std::true_type{}, sa, sb, ks0, vt_last, j, ks1, 0, vt0, 0);
      __syncthreads();
    };
    if constexpr (!scaled) walk(std::false_type{});
    else walk(std::true_type{});
  } else {
    // none of this wave's queries is in the item (the last, partial query
    // tile of a window): it only takes its share of the same tile DMAs and
    // the same nt barriers as the computing waves
    for (int j = 0; j < nt; ++j) {
      const bool even = (j & 1) == 0;
      if (j + 1 < nt) {
        issue_k<D>(even ? ks0 : ks1, min(j + 2, nt - 1), tid, wave_u, nkv, kbase);
        issue_v<D>(even ? vt1 : vt0, j + 1, tid, wave_u, vtbase);
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
      }
      __syncthreads();
    }
  }

  return false;
}

// Normalises the item's outputs and writes them: bf16 rows for tokens one
// window covers (and every dense query), fp32 blend slots for the others.
template <int D, bool WIN>
__device__ __attribute__((always_inline)) inline void epilogue(const AttnArgs& a, const Item& it,
                                                               f32x16 (&o)[kAttnQG][D / 32],
                                                               float (&l_run)[kAttnQG], int ev_cur) {
  constexpr int QG = kAttnQG, BM = kAttnBM, DB = D / 32;
  int qtok[QG];
  bool qvalid[QG];
  query_tokens<WIN>(a, it, qtok, qvalid);
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hi = lane >> 5;
  const int64_t bh = it.bh;
  const int qtile = it.qtile, rec = it.rec, qh = it.qh, qw = it.qw;
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    float lt = pair_sum(l_run[g]);
    float inv = ldexpf(1.0f / lt, ev_cur);
    if (!qvalid[g]) continue;
    const int qt = qtok[g];
    bool direct = true;
    int t = 0;
    if constexpr (WIN) {
      t = qtile * BM + wave * 32 * QG + 32 * g + n;
      int uy = t / qw, ux = t - (t / qw) * qw;
      int wt = min(uy + 1, qh - uy) * min(ux + 1, qw - ux);
      direct = a.wsum[qt] == wt;
    }
    if (direct) {
      u16* orow = a.out + (bh * (int64_t)a.q_rows + a.q0 + qt) * D;
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
  }
}

// The plain kernel: persistent work-groups, one per CU, claim work items
// from per-XCD counters (logical ids contiguous per XCD, so consecutive
// items of a window share its keys in one L2).  After an item's last tile,
// the next item's first tile DMAs are issued before the item's epilogue, so
// their latency overlaps it and no work-group launch separates the items.
template <int D, bool WIN>
__global__ __launch_bounds__(kThreads, kAttnGroupsPerCu) void attn_kernel(const AttnArgs a) {
  // two LDS stages, as separate objects so that the compiler can tell a DMA
  // into one stage from reads of the other
  __shared__ __attribute__((aligned(16))) u16 ks0[BN * D];
  __shared__ __attribute__((aligned(16))) u16 vt0[D * BN];
  __shared__ __attribute__((aligned(16))) u16 ks1[BN * D];
  __shared__ __attribute__((aligned(16))) u16 vt1[D * BN];
  __shared__ int s_sync[kAttnWaves + 1];
  const int xcd = blockIdx.x & 7;
  // logical ids: (batch, head)-major over the call's items, split into 8
  // contiguous shares, one per XCD
  const int64_t total = (WIN ? (int64_t)a.n_items[0] : (int64_t)a.n_qtiles) * a.BH;
  const int per = (int)((total + 7) >> 3);
  int* ctr = a.ctr;
  if (threadIdx.x == 0) s_sync[kAttnWaves] = claim_from(ctr, xcd, per, total, atomicAdd(&ctr[xcd], 1));
  __syncthreads();
  const int first = __builtin_amdgcn_readfirstlane(s_sync[kAttnWaves]);
  __syncthreads();
  if (first < 0) return;
  // pre: the item's first tile DMAs are already in flight at the loop head.
  // Its query loads wait for the loop head: kept in registers across the
  // epilogue they would crowd the key loop's registers.
  int cur = first;
  bool pre = false;
  while (cur >= 0) {
    const Item it = decode_item<D, WIN>(a, cur);
    Queries<D> qs;
    load_queries<D, WIN>(a, it, qs);
    if (!pre) issue_first<D>(it, ks0, vt0, ks1);
    __builtin_amdgcn_sched_barrier(0);  // the DMAs before the rotation's waits
    int fut = 0;
    if ((int)threadIdx.x == 0) fut = atomicAdd(&ctr[xcd], 1);  // the next item, resolved at the item's first barrier
    f32x16 o[kAttnQG][D / 32];
    float l_run[kAttnQG];
    int ev_cur = 0, look = -1;
    const bool listed = compute_item<D, WIN, false>(a, it, qs, ks0, vt0, ks1, vt1, o, l_run, ev_cur, s_sync, ctr,
                                                    xcd, per, total, fut, look);
    pre = false;
    if (!listed) {
      // every LDS stage is free once the key loop's last barrier is passed
      if (look >= 0) {
        issue_first<D>(decode_item<D, WIN>(a, look), ks0, vt0, ks1);
        pre = true;
      }
      epilogue<D, WIN>(a, it, o, l_run, ev_cur);
    }
    cur = look;
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
}

// The scaled kernel: work-groups walk the items the plain kernel listed
// (none for operands within fp16's comfortable range, so it ends at once).
template <int D, bool WIN>
__global__ __launch_bounds__(kThreads, kAttnGroupsPerCu) void attn_scaled_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) u16 ks0[BN * D];
  __shared__ __attribute__((aligned(16))) u16 vt0[D * BN];
  __shared__ __attribute__((aligned(16))) u16 ks1[BN * D];
  __shared__ __attribute__((aligned(16))) u16 vt1[D * BN];
  const int cnt = a.redo[0];
  for (int i = blockIdx.x; i < cnt; i += gridDim.x) {
    const Item it = decode_item<D, WIN>(a, a.redo[1 + i]);
    Queries<D> qs;
    load_queries<D, WIN>(a, it, qs);
    issue_first<D>(it, ks0, vt0, ks1);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 o[kAttnQG][D / 32];
    float l_run[kAttnQG];
    int ev_cur = 0, look = -1;
    compute_item<D, WIN, true>(a, it, qs, ks0, vt0, ks1, vt1, o, l_run, ev_cur, nullptr, nullptr, 0, 0, 0, 0,
                               look);
    epilogue<D, WIN>(a, it, o, l_run, ev_cur);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ blend --
struct BlendArgs {
  int Gh, Gw, D, ny, nx, Ly, Lx;
  int T;               // output rows: T text rows, then the image tokens
  int64_t BH;
  int ys[kMaxAxisWindows], xs[kMaxAxisWindows];
};

constexpr int kBlendTok = 16;
constexpr int kBlendBatch = 4;  // elements per lane whose slot loads are in flight together
constexpr int kMaxCover = 8;

__device__ inline int tent_w(int u, int L) { return min(u + 1, L - u); }

// Tokens covered by more than one window: out = sum_w wt_w * O_w / wsum,
// windows in record order.  One block per kBlendTok tokens: the window
// positions are staged in LDS, the first kBlendTok threads find their
// token's covering rows and columns of windows, then kBlendTok threads per
// token look up one covering window each (its record, quadrant, slot and
// tent weight); finally each wave blends the block's overlapped tokens in
// turn.
__global__ __launch_bounds__(256) void blend_kernel(BlendArgs b, const int32_t* __restrict__ plan,
                                                    const int* __restrict__ rec_start, const int* __restrict__ slot_off,
                                                    const int32_t* __restrict__ wsum, const float* __restrict__ slots,
                                                    u16* __restrict__ out) {
  static_assert(kBlendTok * kBlendTok == 256, "one looker-up per (token, covering window) slot");
  __shared__ int s_ys[kMaxAxisWindows], s_xs[kMaxAxisWindows];
  __shared__ int s_slot[kBlendTok][kMaxCover * kMaxCover];
  __shared__ float s_wt[kBlendTok][kMaxCover * kMaxCover];
  __shared__ int s_cnt[kBlendTok];
  __shared__ int s_cover[kBlendTok][4];  // first covering row window, their count; the same for columns
  __shared__ int s_list[kBlendTok];      // the block's tokens that more than one window covers
  __shared__ int s_nov;
  const int64_t N = (int64_t)b.Gh * b.Gw;
  const int64_t p0 = (int64_t)blockIdx.x * kBlendTok;
  const int tid = threadIdx.x;
  if (tid < b.ny) s_ys[tid] = b.ys[tid];
  if (tid >= kMaxAxisWindows && tid - kMaxAxisWindows < b.nx) s_xs[tid - kMaxAxisWindows] = b.xs[tid - kMaxAxisWindows];
  __syncthreads();
  if (tid < kBlendTok) {
    const int64_t p = p0 + tid;
    int i0 = 0, cy = 0, j0 = 0, cx = 0;
    if (p < N) {
      // window starts along an axis never decrease and all windows of an
      // axis have one length, so a token's covering windows on that axis
      // are consecutive; the first kMaxCover of them are kept
      const int y = (int)p / b.Gw, x = (int)p % b.Gw;
      for (int i = 0; i < b.ny; ++i)
        if (y >= s_ys[i] && y < s_ys[i] + b.Ly && cy < kMaxCover) {
          if (cy == 0) i0 = i;
          ++cy;
        }
      for (int j = 0; j < b.nx; ++j)
        if (x >= s_xs[j] && x < s_xs[j] + b.Lx && cx < kMaxCover) {
          if (cx == 0) j0 = j;
          ++cx;
        }
    }
    s_cover[tid][0] = i0;
    s_cover[tid][1] = cy;
    s_cover[tid][2] = j0;
    s_cover[tid][3] = cx;
    s_cnt[tid] = cy * cx > 1 ? cy * cx : 0;
  }
  __syncthreads();
  {
    const int t = tid / kBlendTok;
    const int64_t p = p0 + t;
    const int cnt = s_cnt[t];
    const int i0 = s_cover[t][0], j0 = s_cover[t][2], cx = s_cover[t][3];
    for (int k = tid % kBlendTok; k < cnt; k += kBlendTok) {
      const int y = (int)p / b.Gw, x = (int)p % b.Gw;
      const int r0 = rec_start[(i0 + k / cx) * b.nx + j0 + k % cx];
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
      const int uy = y - wp[0], ux = x - wp[1];
      s_wt[t][k] = (float)(tent_w(uy, wp[2]) * tent_w(ux, wp[3]));
      s_slot[t][k] = slot_off[rr] + uy * wp[3] + ux;
    }
  }
  if (tid == 0) {
    int n = 0;
    for (int t = 0; t < kBlendTok; ++t)
      if (s_cnt[t] > 1) s_list[n++] = t;
    s_nov = n;
  }
  __syncthreads();
  // Each wave takes the block's overlapped tokens in turn; per token, the
  // (batch*head, 4 channels) elements in batches of kBlendBatch per lane,
  // all of a batch's slot loads in flight together.  32-bit index
  // arithmetic: D/4 is a power of two and BH * D/4 fits an int (checked by
  // the host).
  const int d4_bits = b.D == 128 ? 5 : 4;
  const int per_tok = (int)b.BH << d4_bits;
  const int wave = tid >> 6, lane = tid & 63;
  for (int q = wave; q < s_nov; q += 256 / 64) {
    const int t = s_list[q];
    const int cnt = s_cnt[t];
    const int64_t p = p0 + t;
    const float inv = 1.0f / (float)wsum[p];
    for (int r0 = lane; r0 < per_tok; r0 += 64 * kBlendBatch) {
      float4 acc[kBlendBatch];
#pragma unroll
      for (int k = 0; k < kBlendBatch; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int i = 0; i < cnt; ++i) {
        const float wgt = s_wt[t][i];
        const float* base = slots + (int64_t)s_slot[t][i] * b.BH * b.D;
        float4 v[kBlendBatch];
#pragma unroll
        for (int k = 0; k < kBlendBatch; ++k) {
          const int r = r0 + 64 * k;
          v[k] = r < per_tok ? *reinterpret_cast<const float4*>(base + ((int64_t)(r >> d4_bits) * b.D +
                                                                        4 * (r & ((1 << d4_bits) - 1))))
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < kBlendBatch; ++k) {
          acc[k].x += wgt * v[k].x;
          acc[k].y += wgt * v[k].y;
          acc[k].z += wgt * v[k].z;
          acc[k].w += wgt * v[k].w;
        }
      }
#pragma unroll
      for (int k = 0; k < kBlendBatch; ++k) {
        const int r = r0 + 64 * k;
        if (r >= per_tok) continue;
        const int bh = r >> d4_bits;
        const int c4 = 4 * (r & ((1 << d4_bits) - 1));
        uint2 pk;
        pk.x = (unsigned)f2bf(acc[k].x * inv) | ((unsigned)f2bf(acc[k].y * inv) << 16);
        pk.y = (unsigned)f2bf(acc[k].z * inv) | ((unsigned)f2bf(acc[k].w * inv) << 16);
        *reinterpret_cast<uint2*>(out + ((int64_t)bh * (N + b.T) + b.T + p) * b.D + c4) = pk;
      }
    }
  }
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 256;
    cus[dev] = n / 8 * 8;
  }
  return cus[dev];
}

// work: an upper bound of the call's work items (the window plan's count is
// on the device).
template <bool WIN>
int launch_attn(const AttnArgs& a, int D, int64_t work, hipStream_t st) {
  const AttnArgs& b = a;
  if (work > 0x7FFFFFF0LL) return fail(AREA_E_UNSUPPORTED, "attention work too large");
  const int64_t g = (work + 7) / 8 * 8;
  // the plain kernel is persistent: one work-group per CU slot
  dim3 grid((unsigned)std::min<int64_t>(g, (int64_t)device_cus() * kAttnGroupsPerCu));
  // the scaled kernel's work-groups walk the listed items, one work-group
  // per CU (the register budget of one fits a CU)
  dim3 grid_scaled((unsigned)std::min<int64_t>(g, device_cus()));
  AttnEvents ev = attn_events();
  if (ev.begin) {
    hipError_t e = hipEventRecord((hipEvent_t)ev.begin, st);
    if (e != hipSuccess) return fail(AREA_E_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
  }
  if (D == 128) {
    hipLaunchKernelGGL((attn_kernel<128, WIN>), grid, dim3(kThreads), 0, st, b);
    hipLaunchKernelGGL((attn_scaled_kernel<128, WIN>), grid_scaled, dim3(kThreads), 0, st, b);
  } else {
    hipLaunchKernelGGL((attn_kernel<64, WIN>), grid, dim3(kThreads), 0, st, b);
    hipLaunchKernelGGL((attn_scaled_kernel<64, WIN>), grid_scaled, dim3(kThreads), 0, st, b);
  }
  int rc = check_launch(WIN ? "attn_kernel<window>" : "attn_kernel<dense>");
  if (rc) return rc;
  if (ev.end) {
    hipError_t e = hipEventRecord((hipEvent_t)ev.end, st);
    if (e != hipSuccess) return fail(AREA_E_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
  }
  return AREA_OK;
}

}  // namespace

int launch_kv_tiles(const void* k, const void* v, const void* rope, void* kr, void* vt, int* kexp, int* vexp,
                    int* flags, int64_t BH, int M, int D, bool f32_in, int T, int Gw, stream_t s) {
  if (BH > 65535) return fail(AREA_E_UNSUPPORTED, "batch*heads above 65535");
  const int tiles = (M + BN - 1) / BN;
  if (tiles == 0) return AREA_OK;
  dim3 grid((unsigned)tiles, (unsigned)BH);
  hipStream_t st = (hipStream_t)s;
  const float* tab = (const float*)rope;
  if (D == 128) {
    if (f32_in)
      hipLaunchKernelGGL((kv_tiles_kernel<128, true>), grid, dim3(256), 0, st, k, v, tab, (u16*)kr, (u16*)vt, kexp,
                         vexp, flags, M, tiles, T, Gw);
    else
      hipLaunchKernelGGL((kv_tiles_kernel<128, false>), grid, dim3(256), 0, st, k, v, tab, (u16*)kr, (u16*)vt, kexp,
                         vexp, flags, M, tiles, T, Gw);
  } else {
    if (f32_in)
      hipLaunchKernelGGL((kv_tiles_kernel<64, true>), grid, dim3(256), 0, st, k, v, tab, (u16*)kr, (u16*)vt, kexp,
                         vexp, flags, M, tiles, T, Gw);
    else
      hipLaunchKernelGGL((kv_tiles_kernel<64, false>), grid, dim3(256), 0, st, k, v, tab, (u16*)kr, (u16*)vt, kexp,
                         vexp, flags, M, tiles, T, Gw);
  }
  return check_launch("kv_tiles_kernel");
}

int launch_dense_attn(const void* q, const void* rope, int q_text, int Gh, int Gw, const void* k_rot,
                      const void* vt, const int* kexp, const int* vexp, int* flags, void* out, int64_t BH,
                      int Nq, int q0, int q_rows, int Nk, int D, stream_t s) {
  AttnArgs a = {};
  a.q = (const u16*)q;
  a.rope_P = std::max(Gh, Gw);
  a.rope = (const float4*)rope + (size_t)a.rope_P * (D / 8);  // second table
  a.q_text = q_text;
  a.Gw = Gw;
  a.k = (const u16*)k_rot;
  a.vt = (const u16*)vt;
  a.out = (u16*)out;
  a.BH = BH;
  a.Nq = Nq;
  a.q0 = q0;
  a.q_rows = q_rows;
  a.k_rows = Nk;
  a.k_tiles = (Nk + BN - 1) / BN;
  a.kexp = kexp;
  a.vexp = vexp;
  a.flags = flags;
  a.ctr = flags + BH;
  a.redo = flags + BH + 8;
  a.n_kv = Nk;
  a.n_qtiles = (Nq + kAttnBM - 1) / kAttnBM;
  a.c = (float)(1.4426950408889634 / std::sqrt((double)D));
  if (Nq == 0) return AREA_OK;
  return launch_attn<false>(a, D, (int64_t)a.n_qtiles * BH, (hipStream_t)s);
}

int launch_window_attn(const WindowAttnArgs& w, const int32_t* plan, const int32_t* wsum, const int32_t* bridge_idx,
                       const void* q, const void* k, const void* v, const void* rope, void* out, const WindowWs& ws,
                       stream_t s) {
  // the blend indexes (batch*head, 4 channels) in 32 bits
  if (w.BH * (w.D / 4) > 0x7FFFFFFFLL) return fail(AREA_E_UNSUPPORTED, "blend: batch * heads too large");
  hipStream_t st = (hipStream_t)s;
  int n_base = w.ny * w.nx;
  const int R = bridge_idx ? w.R : 0;
  if (w.BH > 65535) return fail(AREA_E_UNSUPPORTED, "batch*heads above 65535");
  ItemsWs iw = make_items_ws(ws.items, w.max_windows, n_base, w.max_items);
  hipLaunchKernelGGL(items_kernel, dim3(1), dim3(256), 0, st, plan, iw, kAttnBM, R + w.T, w.max_windows,
                     w.max_items, w.max_gtiles);
  int rc = check_launch("items_kernel");
  if (rc) return rc;
  if (R > 0) {
    hipLaunchKernelGGL(bridge_compact_kernel, dim3((unsigned)w.max_windows, (unsigned)w.BH), dim3(256), 0, st, plan,
                       bridge_idx, ws.blist, ws.bcount, R, w.Gw, w.BH);
    rc = check_launch("bridge_compact_kernel");
    if (rc) return rc;
  }
  const int N = w.Gh * w.Gw;
  dim3 gg((unsigned)w.max_gtiles, (unsigned)w.BH);
  if (w.D == 128)
    hipLaunchKernelGGL((gather_kernel<128>), gg, dim3(256), 0, st, plan, (const int*)iw.gtiles, (const int*)iw.n_items,
                       (const int*)iw.kv_tile_off, (const int*)ws.blist, (const int*)ws.bcount, (const u16*)k,
                       (const u16*)v, (const float*)rope, (u16*)ws.kg, (u16*)ws.vg, ws.kexp, ws.vexp, ws.flags,
                       w.max_gtiles, R, w.T, w.Gw, N, w.BH);
  else
    hipLaunchKernelGGL((gather_kernel<64>), gg, dim3(256), 0, st, plan, (const int*)iw.gtiles, (const int*)iw.n_items,
                       (const int*)iw.kv_tile_off, (const int*)ws.blist, (const int*)ws.bcount, (const u16*)k,
                       (const u16*)v, (const float*)rope, (u16*)ws.kg, (u16*)ws.vg, ws.kexp, ws.vexp, ws.flags,
                       w.max_gtiles, R, w.T, w.Gw, N, w.BH);
  rc = check_launch("gather_kernel");
  if (rc) return rc;
  AttnArgs a = {};
  a.q = (const u16*)q;
  a.rope_P = std::max(w.Gh, w.Gw);
  a.rope = (const float4*)rope + (size_t)a.rope_P * (w.D / 8);  // second table
  a.q_text = w.T;
  a.k = (const u16*)ws.kg;
  a.vt = (const u16*)ws.vg;
  a.out = (u16*)out;
  a.BH = w.BH;
  a.Nq = N;
  a.q0 = w.T;
  a.q_rows = w.T + N;
  a.T = w.T;
  a.k_rows = w.max_gtiles * BN;
  a.k_tiles = w.max_gtiles;
  a.kexp = ws.kexp;
  a.vexp = ws.vexp;
  a.flags = ws.flags;
  a.ctr = ws.flags + w.BH;
  a.redo = ws.flags + w.BH + 8;
  a.c = (float)(1.4426950408889634 / std::sqrt((double)w.D));
  a.plan = plan;
  a.wsum = wsum;
  a.items = iw.items;
  a.n_items = iw.n_items;
  a.slot_off = iw.slot_off;
  a.kv_tile_off = iw.kv_tile_off;
  a.bcount = ws.bcount;
  a.slots = ws.slots;
  a.Gw = w.Gw;
  a.R = R;
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
  b.T = w.T;
  b.BH = w.BH;
  for (int i = 0; i < kMaxAxisWindows; ++i) {
    b.ys[i] = w.ys[i];
    b.xs[i] = w.xs[i];
  }
  hipLaunchKernelGGL(blend_kernel, dim3((unsigned)((N + kBlendTok - 1) / kBlendTok)), dim3(256), 0, st, b, plan,
                     (const int*)iw.rec_start, (const int*)iw.slot_off, wsum, (const float*)ws.slots, (u16*)out);
  return check_launch("blend_kernel");
}

}  // namespace area
