// Flash-style attention on gfx950 for the AReA path: full attention, Phase I
// coarse attention over pooled keys, and Phase II windowed attention (Halo
// rectangle + global-KV bridge, tent-weighted blending of overlaps).
//
// Design (CDNA4, wave64):
//  * One attention kernel for every mode.  Its key/value set is always a
//    contiguous run of fp16 K rows plus fp16 V^T tiles of 64 keys: full and
//    coarse attention use the prepared tensors directly, windowed attention
//    first gathers each window's keys (Halo rectangle, then the bridge tokens
//    outside it, compacted; turned by RoPE on the way) with a bandwidth-bound
//    kernel, so no index math or transposition remains in the MFMA loop.
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
//  * Eight waves of 32 queries (256 queries per work-group) use ~240
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
//  * Work items are mapped XCD-aware: consecutive items (same head, same
//    window) land on the same XCD and share its L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <string>

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

__device__ inline u16 bf_to_f16(u16 b) {
  _Float16 h = (_Float16)__uint_as_float(((unsigned)b) << 16);
  return __builtin_bit_cast(u16, h);
}

// Two-axis RoPE of one 16-byte chunk (8 bf16 channels, 4 rotation pairs)
// into fp16: c01, c23 hold the chunk's four (cos, sin) pairs, interleaved.
// Pair (a, b) becomes (a cos - b sin, a sin + b cos) times `scale`, rounded
// to nearest.
__device__ inline u32x4 rope8_f16(const u32x4 raw, const float4 c01, const float4 c23, const float scale = 1.0f) {
  const float co[4] = {c01.x, c01.z, c23.x, c23.z};
  const float sn[4] = {c01.y, c01.w, c23.y, c23.w};
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = __uint_as_float(raw[j] << 16), b = __uint_as_float(raw[j] & 0xFFFF0000u);
    const _Float16 x0 = (_Float16)((a * co[j] - b * sn[j]) * scale);
    const _Float16 x1 = (_Float16)((a * sn[j] + b * co[j]) * scale);
    r[j] = (unsigned)__builtin_bit_cast(u16, x0) | ((unsigned)__builtin_bit_cast(u16, x1) << 16);
  }
  return r;
}

// ------------------------------------------------------------ V^T tiles --
// out[bh][t][d][k] = in[bh][64 t + k][d] as fp16, zero for rows >= M.
template <int D, bool IN_BF16>
__global__ __launch_bounds__(256) void vt_kernel(const u16* __restrict__ in, u16* __restrict__ out, int M,
                                                 int tiles) {
  constexpr int CPR = D / 8;
  constexpr int LS = D + 8;
  __shared__ __attribute__((aligned(16))) u16 buf[BN * LS];
  const int t = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const u16* src = in + bh * (int64_t)M * D;
  for (int c = threadIdx.x; c < BN * CPR; c += 256) {
    int row = c / CPR, col = c - row * CPR;
    int key = t * BN + row;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (key < M) {
      v = *reinterpret_cast<const u32x4*>(src + (int64_t)key * D + col * 8);
      if constexpr (IN_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = (unsigned)bf_to_f16((u16)(v[i] & 0xFFFFu)) | ((unsigned)bf_to_f16((u16)(v[i] >> 16)) << 16);
      }
    }
    *reinterpret_cast<u32x4*>(buf + row * LS + col * 8) = v;
  }
  __syncthreads();
  u16* dst = out + (bh * tiles + t) * (int64_t)D * BN;
  for (int c = threadIdx.x; c < D * (BN / 8); c += 256) {
    int d = c / (BN / 8), k8 = c - d * (BN / 8);
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = (unsigned)buf[(8 * k8 + 2 * i) * LS + d] | ((unsigned)buf[(8 * k8 + 2 * i + 1) * LS + d] << 16);
    *reinterpret_cast<u32x4*>(dst + d * BN + 8 * k8) = v;
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
// sin) table `rope` and written as fp16; V rows are converted bf16 -> fp16
// and written transposed.
template <int D>
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ plan, const int* __restrict__ gtiles,
                                                     const int* __restrict__ n_items, const int* __restrict__ kv_tile_off,
                                                     const int* __restrict__ list, const int* __restrict__ count,
                                                     const u16* __restrict__ k, const u16* __restrict__ v,
                                                     const float* __restrict__ rope, u16* __restrict__ kg,
                                                     u16* __restrict__ vg, int64_t cap_tiles, int R, int Tt, int Gw,
                                                     int N, int64_t BH) {
  constexpr int CPR = D / 8;
  constexpr int HALF = CPR / 2;  // chunks per axis half
  constexpr int NF = D / 4;      // frequencies per axis half
  constexpr int LS = D + 8;
  __shared__ __attribute__((aligned(16))) u16 buf[BN * LS];
  __shared__ int s_tok[BN];
  __shared__ int s_py[BN], s_px[BN];
  const int g = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (g >= n_items[1]) return;
  const int rec = gtiles[2 * g], t = gtiles[2 * g + 1];
  const int32_t* rp = plan + AREA_PLAN_HEADER + AREA_PLAN_REC * rec;
  const int ky0 = rp[4], kx0 = rp[5], kw = rp[7];
  const int nrect = rp[6] * kw;
  const int cnt = R > 0 ? count[(int64_t)rec * BH + bh] : 0;
  const int T = kv_tile_off[rec] + t;
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
  u16* kdst = kg + (bh * cap_tiles + T) * (int64_t)BN * D;
  for (int c = threadIdx.x; c < BN * CPR; c += 256) {
    int row = c / CPR, col = c - row * CPR;
    int tok = s_tok[row];
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (tok >= 0) {
      // chunk col: channels 8 col .. 8 col + 7, rotation pairs 4 (col % HALF) ..
      // of the row (first half) or column (second half) axis
      const int pos = col < HALF ? s_py[row] : s_px[row];
      const float4* cs = reinterpret_cast<const float4*>(rope + 2 * (pos * NF + 4 * (col % HALF)));
      kv = rope8_f16(*reinterpret_cast<const u32x4*>(ksrc + (int64_t)tok * D + col * 8), cs[0], cs[1]);
      vv = *reinterpret_cast<const u32x4*>(vsrc + (int64_t)tok * D + col * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vv[i] = (unsigned)bf_to_f16((u16)(vv[i] & 0xFFFFu)) | ((unsigned)bf_to_f16((u16)(vv[i] >> 16)) << 16);
    }
    *reinterpret_cast<u32x4*>(kdst + row * D + col * 8) = kv;
    *reinterpret_cast<u32x4*>(buf + row * LS + col * 8) = vv;
  }
  __syncthreads();
  u16* vdst = vg + (bh * cap_tiles + T) * (int64_t)D * BN;
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
  int n_kv;            // dense mode: keys per query
  int n_qtiles;        // dense mode: query tiles per head
  int grid;            // launched work-groups (multiple of 8)
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
template <int D, int QG>
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
    const f16x8 f = fr[j % PF];
    if (j + PF < NT) fr[j % PF] = lds_frag(ks, k_frag_off<D>(j + PF, n, hi));
    else vfr[j + PF - NT] = lds_frag(vt, vt_frag_off<D>(j + PF - NT, n, hi));
#pragma unroll
    for (int g = 0; g < QG; ++g)
      sn[g][j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f, qf[g][j >> 1], j < 2 ? nm[g] : sn[g][j & 1], 0, 0, 0);
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

template <int D, bool WIN>
__global__ __launch_bounds__(kThreads, kAttnGroupsPerCu) void attn_kernel(const AttnArgs a) {
  constexpr int QG = kAttnQG;     // 32-query groups per wave
  constexpr int BM = kAttnBM;     // kAttnWaves waves x QG groups x 32 queries
  constexpr int KD = D / 16;
  constexpr int DB = D / 32;
  constexpr int K_ELEMS = BN * D;
  constexpr int V_ELEMS = D * BN;
  static_assert(BM == kAttnWaves * 32 * QG, "query tile");

  // two LDS stages, as separate objects so that the compiler can tell a DMA
  // into one stage from reads of the other
  __shared__ __attribute__((aligned(16))) u16 ks0[K_ELEMS];
  __shared__ __attribute__((aligned(16))) u16 vt0[V_ELEMS];
  __shared__ __attribute__((aligned(16))) u16 ks1[K_ELEMS];
  __shared__ __attribute__((aligned(16))) u16 vt1[V_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hi = lane >> 5;

  // ---- work item (XCD-aware order: logical ids are contiguous per XCD)
  const int pid = blockIdx.x;
  const int64_t L = (int64_t)(pid & 7) * (a.grid >> 3) + (pid >> 3);
  int64_t bh;
  int qtile = 0, rec = 0;
  int qy0 = 0, qx0 = 0, qh = 0, qw = 1;
  int nq, nkv;
  int64_t t0 = 0;  // first key tile of the item's key set
  if constexpr (WIN) {
    bh = L / a.max_items;
    int64_t it = L - bh * a.max_items;
    if (bh >= a.BH || it >= a.n_items[0]) return;
    rec = a.items[2 * it];
    qtile = a.items[2 * it + 1];
    const int32_t* rp = a.plan + AREA_PLAN_HEADER + AREA_PLAN_REC * rec;
    qy0 = rp[0]; qx0 = rp[1]; qh = rp[2]; qw = rp[3];
    nq = qh * qw;
    nkv = rp[6] * rp[7] + (a.R > 0 ? a.bcount[(int64_t)rec * a.BH + bh] : 0) + a.T;
    t0 = a.kv_tile_off[rec];
  } else {
    bh = L / a.n_qtiles;
    qtile = (int)(L - bh * a.n_qtiles);
    if (bh >= a.BH) return;
    nq = a.Nq;
    nkv = a.n_kv;
  }
  const u16* kbase = a.k + bh * a.k_rows * D + t0 * BN * D;
  const u16* vtbase = a.vt + (bh * a.k_tiles + t0) * (int64_t)D * BN;
  const u16* qbase = a.q + (bh * (int64_t)a.q_rows + a.q0) * D;

  // ---- queries of this lane
  int qtok[QG];
  bool qvalid[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    int t = qtile * BM + wave * 32 * QG + 32 * g + n;
    qvalid[g] = t < nq;
    if constexpr (WIN) {
      int yy = qvalid[g] ? t / qw : 0;
      int xx = qvalid[g] ? t - yy * qw : 0;
      qtok[g] = (qy0 + yy) * a.Gw + qx0 + xx;
    } else {
      qtok[g] = qvalid[g] ? t : 0;
    }
  }
  // MFMA B operand: chunk 2 kd + hi (channels 16 kd + 8 hi ..) of the
  // lane's query, turned by RoPE at its grid position (chunks of the first
  // half follow the row, the others the column; text rows sit at (0, 0)).
  // The raw chunks and their (cos, sin) are loaded here and turned after
  // the first tile DMAs have been started, so the two latencies overlap.
  u32x4 qraw[QG][KD];
  float4 qcs[QG][KD][2];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int64_t row = (int64_t)a.q0 + qtok[g];
    int py = 0, px = 0;
    if (row >= a.q_text) {
      const int img = (int)(row - a.q_text);
      py = img / a.Gw;
      px = img - py * a.Gw;
    }
    const u32x4* qrow = reinterpret_cast<const u32x4*>(qbase + (int64_t)qtok[g] * D);
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const int ch = 2 * kd + hi;
      const int pos = kd < KD / 2 ? py : px;
      // frequencies 4 (ch % KD) .. + 3: pairs 2 (ch % KD) and 2 (ch % KD) + 1
      const float4* cs = a.rope + (int64_t)(2 * (ch % KD)) * a.rope_P + pos;
      qraw[g][kd] = qrow[ch];
      qcs[g][kd][0] = cs[0];
      qcs[g][kd][1] = cs[a.rope_P];
    }
  }
  f16x8 qf[QG][KD];

  const int nt = (nkv + BN - 1) / BN;
  const float c = a.c;

  f32x16 o[QG][DB];
  f32x16 nm[QG];  // -m, the running maximum (log2 units), in all 16 registers
  float l_run[QG];
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
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // the buffer resources below need wave-uniform bases and sizes
  kbase = uniform_ptr(kbase);
  vtbase = uniform_ptr(vtbase);
  nkv = __builtin_amdgcn_readfirstlane(nkv);
  auto step = [&](f32x16 (&scur)[QG][2], f32x16 (&snext)[QG][2], const u16* ksn, const u16* vtc, int j,
                  u16* kdma, int ktile, u16* vdma, int vtile)
      __attribute__((always_inline)) {
    // phase A's first K fragments, read ahead of the tile DMAs so their LDS
    // latency overlaps them
    f16x8 kfr[kFragAhead];
#pragma unroll
    for (int jj = 0; jj < kFragAhead; ++jj)
      kfr[jj] = lds_frag(ksn, k_frag_off<D>(jj, n, hi));
    __builtin_amdgcn_sched_barrier(0);
    // DMAs of the next tiles into the two free stages
    issue_k<D>(kdma, ktile, tid, wave_u, nkv, kbase);
    issue_v<D>(vdma, vtile, tid, wave_u, vtbase);
    f16x8 pf[QG][4];
    f16x8 vfr[kFragAhead];
    float psum[QG];
    phase_a<D, QG>(snext, ksn, n, hi, qf, scur, nm, pf, kfr, vtc, vfr, psum);
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
          snext[g][0][i] -= dlt;
          snext[g][1][i] -= dlt;
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
    if (valid < BN) mask_tail<QG>(snext, valid, hi);
    phase_b<D, QG>(o, vtc, n, hi, pf, vfr);
#pragma unroll
    for (int g = 0; g < QG; ++g) l_run[g] += psum[g];
  };

  // Stage use: K tile t in ks[t % 2], V tile t in vt[t % 2].  Each step
  // reads its first K fragments, starts the DMAs into the two free stages,
  // computes, then waits for its own DMAs and syncs.  No DMA is outstanding
  // at a branch merge; the last half-iteration re-loads clamped tiles instead
  // of branching around the DMA, and its scores of the tile past the end are
  // never used.
  f32x16 sa[QG][2], sb[QG][2];
  issue_k<D>(ks0, 0, tid, wave_u, nkv, kbase);
  issue_v<D>(vt0, 0, tid, wave_u, vtbase);
  issue_k<D>(ks1, min(1, nt - 1), tid, wave_u, nkv, kbase);
  __builtin_amdgcn_sched_barrier(0);  // all three DMAs before the rotation's waits
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
      qf[g][kd] = __builtin_bit_cast(f16x8, rope8_f16(qraw[g][kd], qcs[g][kd][0], qcs[g][kd][1], c));
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  tile_scores<D, QG>(sa, ks0, n, hi, qf);
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
  for (int g = 0; g < QG; ++g) any_q |= qvalid[g];
  if (__any(any_q)) {
    for (int j = 0; j < nt; j += 2) {
      step(sa, sb, ks1, vt0, j, ks0, min(j + 2, nt - 1), vt1, min(j + 1, nt - 1));
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();
      if (j + 1 >= nt) break;
      step(sb, sa, ks0, vt1, j + 1, ks1, min(j + 3, nt - 1), vt0, min(j + 2, nt - 1));
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();
    }
  } else {
    // none of this wave's queries is in the item (the last, partial query
    // tile of a window): it only takes its share of the same tile DMAs and
    // the same nt barriers as the computing waves
    for (int j = 0; j < nt; ++j) {
      const bool even = (j & 1) == 0;
      issue_k<D>(even ? ks0 : ks1, min(j + 2, nt - 1), tid, wave_u, nkv, kbase);
      issue_v<D>(even ? vt1 : vt0, min(j + 1, nt - 1), tid, wave_u, vtbase);
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();
    }
  }

  // ---- epilogue: normalise and write
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    float lt = pair_sum(l_run[g]);
    float inv = 1.0f / lt;
    if (!qvalid[g]) continue;
    // an opaque copy of the query's row: its addresses are recomputed here
    // rather than kept live in registers across the key loop
    int qt = qtok[g];
    asm volatile("" : "+v"(qt));
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

// ------------------------------------------------------------------ blend --
struct BlendArgs {
  int Gh, Gw, D, ny, nx, Ly, Lx;
  int T;               // output rows: T text rows, then the image tokens
  int64_t BH;
  int ys[kMaxAxisWindows], xs[kMaxAxisWindows];
};

constexpr int kBlendTok = 16;
constexpr int kMaxCover = 8;

__device__ inline int tent_w(int u, int L) { return min(u + 1, L - u); }

// Tokens covered by more than one window: out = sum_w wt_w * O_w / wsum,
// windows in record order.  One block per kBlendTok tokens: the first
// kBlendTok threads find their token's covering windows in parallel, then
// the whole block writes the blended rows of the overlapped ones.
__global__ __launch_bounds__(256) void blend_kernel(BlendArgs b, const int32_t* __restrict__ plan,
                                                    const int* __restrict__ rec_start, const int* __restrict__ slot_off,
                                                    const int32_t* __restrict__ wsum, const float* __restrict__ slots,
                                                    u16* __restrict__ out) {
  __shared__ int s_slot[kBlendTok][kMaxCover * kMaxCover];
  __shared__ float s_wt[kBlendTok][kMaxCover * kMaxCover];
  __shared__ int s_cnt[kBlendTok];
  const int64_t N = (int64_t)b.Gh * b.Gw;
  const int64_t p0 = (int64_t)blockIdx.x * kBlendTok;
  if (threadIdx.x < kBlendTok) {
    const int t = threadIdx.x;
    const int64_t p = p0 + t;
    int cnt = 0;
    if (p < N) {
      const int y = (int)(p / b.Gw), x = (int)(p % b.Gw);
      int iy[kMaxCover], ix[kMaxCover], cy = 0, cx = 0;
      for (int i = 0; i < b.ny; ++i)
        if (y >= b.ys[i] && y < b.ys[i] + b.Ly && cy < kMaxCover) iy[cy++] = i;
      for (int j = 0; j < b.nx; ++j)
        if (x >= b.xs[j] && x < b.xs[j] + b.Lx && cx < kMaxCover) ix[cx++] = j;
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
            s_wt[t][cnt] = (float)(tent_w(uy, wp[2]) * tent_w(ux, wp[3]));
            s_slot[t][cnt] = slot_off[rr] + uy * wp[3] + ux;
            ++cnt;
          }
      }
    }
    s_cnt[t] = cnt;
  }
  __syncthreads();
  const int D4 = b.D / 4;
  const int64_t per_tok = b.BH * D4;
  for (int64_t e = threadIdx.x; e < kBlendTok * per_tok; e += blockDim.x) {
    const int t = (int)(e / per_tok);
    const int cnt = s_cnt[t];
    if (cnt <= 1) continue;
    const int64_t r = e - t * per_tok;
    const int64_t bh = r / D4;
    const int d4 = (int)(r - bh * D4);
    const int64_t p = p0 + t;
    const float inv = 1.0f / (float)wsum[p];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 0; i < cnt; ++i) {
      float4 v = *reinterpret_cast<const float4*>(slots + ((int64_t)s_slot[t][i] * b.BH + bh) * b.D + 4 * d4);
      float wgt = s_wt[t][i];
      acc.x += wgt * v.x;
      acc.y += wgt * v.y;
      acc.z += wgt * v.z;
      acc.w += wgt * v.w;
    }
    uint2 pk;
    pk.x = (unsigned)f2bf(acc.x * inv) | ((unsigned)f2bf(acc.y * inv) << 16);
    pk.y = (unsigned)f2bf(acc.z * inv) | ((unsigned)f2bf(acc.w * inv) << 16);
    *reinterpret_cast<uint2*>(out + (bh * (N + b.T) + b.T + p) * b.D + 4 * d4) = pk;
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
    hipLaunchKernelGGL((attn_kernel<128, WIN>), grid, dim3(kThreads), 0, st, b);
  else
    hipLaunchKernelGGL((attn_kernel<64, WIN>), grid, dim3(kThreads), 0, st, b);
  int rc = check_launch(WIN ? "attn_kernel<window>" : "attn_kernel<dense>");
  if (rc) return rc;
  if (ev.end) {
    hipError_t e = hipEventRecord((hipEvent_t)ev.end, st);
    if (e != hipSuccess) return fail(AREA_E_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
  }
  return AREA_OK;
}

}  // namespace

size_t vt_bytes(int64_t BH, int M, int D) { return (size_t)BH * ((M + BN - 1) / BN) * BN * D * 2; }

int launch_vt(const void* v, void* vt, int64_t BH, int M, int D, bool bf16_in, stream_t s) {
  if (BH > 65535) return fail(AREA_E_UNSUPPORTED, "batch*heads above 65535");
  int tiles = (M + BN - 1) / BN;
  dim3 grid((unsigned)tiles, (unsigned)BH);
  hipStream_t st = (hipStream_t)s;
  if (D == 128) {
    if (bf16_in) hipLaunchKernelGGL((vt_kernel<128, true>), grid, dim3(256), 0, st, (const u16*)v, (u16*)vt, M, tiles);
    else hipLaunchKernelGGL((vt_kernel<128, false>), grid, dim3(256), 0, st, (const u16*)v, (u16*)vt, M, tiles);
  } else {
    if (bf16_in) hipLaunchKernelGGL((vt_kernel<64, true>), grid, dim3(256), 0, st, (const u16*)v, (u16*)vt, M, tiles);
    else hipLaunchKernelGGL((vt_kernel<64, false>), grid, dim3(256), 0, st, (const u16*)v, (u16*)vt, M, tiles);
  }
  return check_launch("vt_kernel");
}

int launch_dense_attn(const void* q, const void* rope, int q_text, int Gh, int Gw, const void* k_rot,
                      const void* vt, void* out, int64_t BH, int Nq, int q0, int q_rows, int Nk, int D, stream_t s) {
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
  a.n_kv = Nk;
  a.n_qtiles = (Nq + kAttnBM - 1) / kAttnBM;
  a.c = (float)(1.4426950408889634 / std::sqrt((double)D));
  if (Nq == 0) return AREA_OK;
  return launch_attn<false>(a, D, (int64_t)a.n_qtiles * BH, (hipStream_t)s);
}

size_t window_items_ws_bytes(int max_windows, int64_t max_items, int n_base, int64_t max_gtiles) {
  return align_up(2 * sizeof(int)) + 2 * align_up(sizeof(int) * (max_windows > 0 ? max_windows : 1)) +
         align_up(sizeof(int) * (n_base > 0 ? n_base : 1)) + align_up(sizeof(int) * 2 * (max_items > 0 ? max_items : 1)) +
         align_up(sizeof(int) * 2 * (max_gtiles > 0 ? max_gtiles : 1));
}

int launch_window_attn(const WindowAttnArgs& w, const int32_t* plan, const int32_t* wsum, const int32_t* bridge_idx,
                       const void* q, const void* k, const void* v, const void* rope, void* out, const WindowWs& ws,
                       stream_t s) {
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
                       (const u16*)v, (const float*)rope, (u16*)ws.kg, (u16*)ws.vg, w.max_gtiles, R, w.T, w.Gw, N,
                       w.BH);
  else
    hipLaunchKernelGGL((gather_kernel<64>), gg, dim3(256), 0, st, plan, (const int*)iw.gtiles, (const int*)iw.n_items,
                       (const int*)iw.kv_tile_off, (const int*)ws.blist, (const int*)ws.bcount, (const u16*)k,
                       (const u16*)v, (const float*)rope, (u16*)ws.kg, (u16*)ws.vg, w.max_gtiles, R, w.T, w.Gw, N,
                       w.BH);
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
