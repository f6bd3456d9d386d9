/*
 * area.h -- C ABI of the adaptive receptive-field attention (AReA) library
 * for AMD Instinct MI355X (gfx950).
 *
 * AReA replaces uniform full self-attention of a diffusion transformer above
 * its native resolution with a receptive field that narrows over the
 * denoising steps ("AReA: Adaptive Receptive-Field Attention for Efficient
 * High-Resolution Diffusion Transformers", ai.info summary, section
 * "Methodology in Plain English"; AReA README introduction):
 *   Phase I  -- full-resolution queries attend to keys/values pooled one
 *               token per f x f block onto a near-native grid
 *               (area_pool_kv + area_coarse_attn);
 *   Phase II -- queries attend inside shrinking windows, split over smooth
 *               regions of a Haar detail map, widened by a Halo and joined
 *               by a global-KV bridge, with centre-weighted blending of
 *               overlaps (area_dwt_detail + area_window_plan +
 *               area_window_attn).
 * area_full_attn is uniform full attention at the same shape, the
 * baseline the method's speedup is quoted against.
 *
 * Conventions shared by every call
 * --------------------------------
 *  * Tensors are caller-owned, contiguous DEVICE buffers.  Q, K, V and the
 *    outputs are bfloat16 laid out [B][H][T+Gh*Gw][D] (token sequences,
 *    below); image token n sits at grid row y = n / Gw, column x = n % Gw.
 *    Q and K are passed WITHOUT
 *    rotary embedding: the library rotates them itself (two-axis RoPE: the
 *    first D/2 channels encode y, the last D/2 encode x, channel pair
 *    (2k, 2k+1) of an axis half turns by pos * theta^(-4k/D)).
 *  * The attention MFMAs take IEEE fp16 operands (rotated Q and K, V and
 *    the probabilities P; three mantissa bits finer than bf16, same rate)
 *    with fp32 accumulation; the library converts keys and values into
 *    workspace and queries in registers as they are loaded.  Range policy:
 *    fp16 ends at 65504 while bf16 reaches 3e38, so every 64-key tile of K
 *    and of V, and every query row, is stored at its own power-of-two scale
 *    2^-e: e = 0 (the values unchanged) while the block's largest magnitude
 *    lies in [2^-8, 2^15), otherwise chosen so that it lands in
 *    [2^13, 2^14).  Work items that meet a nonzero e run a second attention
 *    kernel that undoes the scales in fp32 (O is kept in the units of the
 *    largest V scale met so far, so P never exceeds fp16).  Any finite input
 *    with |q| |k| sqrt(D) < 2^100 and |v| < 2^100 is handled at the
 *    relative precision of unit-scale data; the bridge's mean key saturates
 *    keys at 2^28.  Inputs holding inf or NaN give undefined outputs.
 *  * The library never allocates device memory.  Calls that need scratch
 *    take a caller-provided workspace of at least area_workspace_bytes()
 *    bytes (device memory, 256-byte aligned).
 *  * Every device call validates its arguments on the host first; on any
 *    error it returns a negative status and launches nothing.  On success
 *    it only enqueues kernels on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns without synchronising.  The computing calls
 *    (area_pool_kv through area_attn_step) allocate and copy nothing and
 *    clear words only with their own kernels (no hipMemset), so a caller
 *    may capture them (a whole step included) into a HIP graph and replay
 *    it.  A failed launch returns
 *    AREA_E_HIP.  area_last_error() gives a per-thread description of the
 *    last failure.
 *  * Calls are re-entrant.  The only process state is the thread-local
 *    error text and measurement events, a per-device cache of the CU
 *    count, and the per-device scratch of area_window_plan_static.  Two
 *    calls that share an output or workspace buffer must be ordered by the
 *    caller (same stream or events).
 */
#ifndef AREA_H
#define AREA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define AREA_OK             0
#define AREA_E_INVALID     -1  /* null pointer, bad enum, negative size          */
#define AREA_E_SHAPE       -2  /* grid / factor / window / bridge inconsistency  */
#define AREA_E_UNSUPPORTED -3  /* valid request outside what is implemented      */
#define AREA_E_WORKSPACE   -4  /* workspace missing or too small                 */
#define AREA_E_HIP         -5  /* a HIP runtime call or kernel launch failed     */

/* ---- enums ------------------------------------------------------------- */
#define AREA_POOL_MEAN   0     /* average of the f x f block                    */
#define AREA_POOL_CENTER 1     /* token at offset (f/2, f/2) of the block       */
#define AREA_POOL_MEDOID 2     /* block token with the least summed key distance */
#define AREA_POOL_RANDOM 3     /* seeded random token of the block              */

#define AREA_PHASE_FULL   0    /* canvas at or below native: keep full attention */
#define AREA_PHASE_COARSE 1    /* Phase I step                                   */
#define AREA_PHASE_WINDOW 2    /* Phase II step                                  */

#define AREA_OP_FULL   0       /* workspace selectors for area_workspace_bytes */
#define AREA_OP_COARSE 1
#define AREA_OP_PLAN   2
#define AREA_OP_WINDOW 3
#define AREA_OP_STEP   4       /* area_attn_step: every intermediate of one step */

/* Plan buffer layout (int32): AREA_PLAN_HEADER header words, then up to
 * max_windows records of AREA_PLAN_REC words each. */
#define AREA_PLAN_HEADER 16
#define AREA_PLAN_REC    10
/* header word indices */
#define AREA_PH_NWIN   0       /* windows after quadrant splits                 */
#define AREA_PH_STEP   1       /* Phase II step index                           */
#define AREA_PH_W      2       /* scheduled window side                         */
#define AREA_PH_NY     3       /* base windows along y                          */
#define AREA_PH_NX     4       /* base windows along x                          */
#define AREA_PH_JITY   5       /* boundary shift applied along y                */
#define AREA_PH_JITX   6       /* boundary shift applied along x                */
#define AREA_PH_HALO   7       /* Halo width (its maximum when drawn per window) */
#define AREA_PH_R      8       /* bridge tokens per (batch, head); 0 = none     */
#define AREA_PH_NSPLIT 9       /* base windows that were split                  */
#define AREA_PH_QTOT  10       /* sum of query-rect areas over all windows      */
/* record fields: qy0 qx0 qh qw  ky0 kx0 kh kw  parent quadrant(-1 | 0..3) */

/* ---- token sequences ----------------------------------------------------
 * Every q, k, v and out tensor is [B][H][T + Gh*Gw][D]: T text tokens first,
 * then the image tokens in row-major order (image token (y, x) is row
 * T + y*Gw + x).  Text tokens sit at RoPE position (0, 0), i.e. are not
 * rotated; pooling leaves them out (ai.info summary, Methodology, Phase I:
 * an image query's key set is the T text keys plus N/f^2 pooled keys) and join every
 * Phase II key set whole.  The image-query calls (area_coarse_attn,
 * area_window_attn) write the image rows of out; text queries take the dense
 * path over all T + N keys (area_text_attn).  area_full_attn writes every
 * row.  T = 0 gives the image-only layout [B][H][Gh*Gw][D]. */

/* ---- problem description ------------------------------------------------ */
typedef struct area_problem {
  int32_t B, H, D;            /* batch, heads, head dim (64 or 128)              */
  int32_t Gh, Gw;             /* image token grid (rows, columns)                */
  int32_t native_h, native_w; /* the model's native token grid                   */
  int32_t T;                  /* text tokens ahead of the image tokens (0 = none) */
  float   rope_theta;         /* RoPE base, e.g. 10000                           */
  int32_t p1_steps;           /* Phase I (coarse) steps                          */
  int32_t f0;                 /* first pooling factor; 0 = derive from native    */
  int32_t f_min;              /* pooling floor (2)                               */
  int32_t pool_mode;          /* AREA_POOL_MEAN | _CENTER | _MEDOID | _RANDOM    */
  int32_t p2_steps;           /* Phase II (window) steps                         */
  int32_t w_start, w_min;     /* window side at the first / last Phase II step;  */
                              /* w_start 0 = derive (largest even side whose     */
                              /* tiling costs fewer pairs than full attention)   */
  int32_t halo;               /* Halo width in tokens (when halo_max == 0)       */
  int32_t bridge_k;           /* bridge tokens per (batch, head) when            */
                              /* bridge_rho_num == 0; 0 = no bridge              */
  int32_t split_num, split_den; /* smooth-window threshold (1/2)                 */
  uint64_t seed;              /* seeds the window-boundary shift and the Halo    */
                              /* widths                                          */
  int32_t halo_max;           /* > 0: every window draws its Halo width from     */
                              /* 1..halo_max (seeded); 0: fixed width `halo`     */
  int32_t bridge_rho_num, bridge_rho_den; /* num > 0: the bridge of window step  */
                              /* t has R_t = round(rho w_t)^2 tokens, rho =      */
                              /* num/den; 0: bridge_k at every step              */
} area_problem;

typedef struct area_step {
  int32_t phase;              /* AREA_PHASE_*                                    */
  int32_t f;                  /* pooling factor of a coarse step, else 0        */
  int32_t w;                  /* window side of a window step, else 0           */
  int32_t ny, nx;             /* base windows per axis                           */
  int32_t jit_y, jit_x;       /* boundary shift per axis                         */
  int32_t max_windows;        /* upper bound on windows after splits (4 ny nx)   */
  int64_t q_total;            /* sum of base-window query areas                  */
  int32_t R;                  /* bridge tokens per (batch, head) of a window     */
                              /* step (0: none), else 0                          */
  int32_t bridge_rh, bridge_rw; /* the bridge's cell grid (R = rh * rw cells,    */
                              /* the most nearly square cells in tokens); 0, 0   */
                              /* without a bridge                                */
} area_step;

/* ---- host-only calls (no GPU needed) ------------------------------------ */

/* Checks a problem: sizes positive, D in {64, 128}, 0 <= T <= 2^20, both grid sides
 * even and at most 65536 (AREA_E_UNSUPPORTED above), T + Gh*Gw <= 2^30 and
 * B*H*(T + Gh*Gw)*D <= 2^40, a common factor >= max(2, f_min) when the canvas exceeds native
 * (README canvas rules), w_min <= w_start, window sides even and >= 2,
 * bridge cells fit the grid, split_den > 0.  Returns AREA_OK or an error. */
int area_validate(const area_problem* p);

/* Phase and schedule of denoising step `step` (0-based, Phase I steps
 * first): the pooling factor from the linear ramp f0 -> f_min snapped to
 * common grid divisors (blog, "Las dos fases de AReA", Fase I, with the
 * worked example at 4096^2), or the window side from the geometric shrink
 * w_start -> w_min, the base tiling counts and the step's boundary shift
 * (ai.info summary, Methodology, Phase II).  At or below native every step
 * is AREA_PHASE_FULL. */
int area_step_info(const area_problem* p, int step, area_step* out);

/* Phase I step count from a sampler's noise schedule (ai.info summary,
 * Scheduling the switch; README sigma* paragraph: the switch is a noise
 * level sigma*, 0.86 .. 0.96 for the tuned models, not a step count).
 * sigmas[0 .. n_steps-1] are the noise levels of the denoising steps in
 * order; *p1_steps receives the number of leading steps with
 * sigmas[t] > sigma_star (the first step at or below sigma_star starts
 * Phase II, later steps stay there).  Use it as area_problem.p1_steps and
 * n_steps - *p1_steps as p2_steps.  Host only.  Returns AREA_OK, or
 * AREA_E_INVALID for NULL pointers, n_steps < 0 or a NaN sigma_star. */
int area_phase1_steps_for_sigma(const double* sigmas, int n_steps, double sigma_star, int* p1_steps);

/* First pooling factor (f0 from the problem, or derived from the native
 * grid when p->f0 == 0).  Returns the factor or a negative status. */
int area_f0(const area_problem* p);

/* Base windows of Phase II step `step` (before quadrant splits) as
 * (y0, x0, h, w) int32 quadruples in row-major order, written to the HOST
 * array out[4 * cap].  Returns the window count, or a negative status
 * (AREA_E_INVALID if cap is too small). */
int area_base_windows(const area_problem* p, int step, int32_t* out, int cap);

/* Bytes of device workspace needed by the calls of class `op`
 * (AREA_OP_*), the maximum over all steps of the problem.  0 on error. */
size_t area_workspace_bytes(const area_problem* p, int op);

/* int32 words of the plan buffer for any step of the problem. */
size_t area_plan_words(const area_problem* p);

/* Measurement hook for tracing (not needed for computing).  While set on
 * the calling thread, every attention-kernel launch of a device call
 * (area_full_attn, area_coarse_attn, area_window_attn) records the HIP event
 * `ev_begin` just before the kernel and `ev_end` just after it, on the
 * call's stream, so a profiler-free caller can time the MFMA kernel alone
 * (without the key preparation, gather and blend kernels around it; the
 * queries' RoPE and fp16 conversion run inside the kernel).  Events
 * are hipEvent_t handles owned by the caller; pass NULL, NULL to clear.
 * Thread-local; returns AREA_OK, or AREA_E_INVALID if exactly one is NULL. */
int area_set_attn_events(void* ev_begin, void* ev_end);

/* Measurement hook (not needed for computing): the fp16/bf16 matrix-core
 * rate the current device sustains.  Launches a register-only stream of
 * v_mfma_f32_32x32x16_f16 (eight 256-thread work-groups per CU, four
 * independent accumulators per wave, no memory traffic) twice on `stream`,
 * times the second launch with HIP events and returns TFLOP/s in *tflops,
 * the ceiling that the attention kernels are compared with next to the
 * published peak (the shader clock under load sits below nominal).
 * Synchronises `stream`.  `sink` is a caller-owned device buffer of at least
 * 4 bytes; the kernel's only store to it sits under a condition that cannot
 * hold, so it is never written.  Returns AREA_OK, AREA_E_INVALID if a pointer
 * is NULL, or AREA_E_HIP. */
int area_measure_mfma_peak(void* sink, double* tflops, void* stream);

/* Human-readable text for a status, and the thread's last error detail. */
const char* area_strerror(int status);
const char* area_last_error(void);

/* ---- device calls ------------------------------------------------------- */

/* Phase I pooling (blog Fase I; ai.info summary Phase I; README Phase I
 * bullet).  k, v: [B][H][T+Gh*Gw][D] bf16, un-rotated.  kp, vp: outputs
 * [B][H][T+(Gh/f)*(Gw/f)][D] in fp32 (the pooled means unrounded, and the
 * inputs' full range kept; area_coarse_attn converts them to its fp16
 * operands).  Block (by, bx) sits at index by*(Gw/f)+bx.
 * kp = RoPE(pool(k)) at integer coarse position (by, bx); vp = pool(v).
 * pool per p->pool_mode (blog "Cómo entra en tu pipeline": the pooling
 * tunable takes subsample, mean, medoid or random): the mean of the block's
 * f*f tokens (fp32 sum, one fp32 division), or one token of the block, the same
 * token for K and V: the block centre (offset (f/2, f/2)); the medoid (the
 * token whose un-rotated key has the smallest sum of Euclidean distances to
 * the block's keys, float64, per pair the squared differences summed over
 * d ascending, then the square roots summed over the other token ascending;
 * ties to the smaller row-major offset; per batch and head); or a random
 * token, offset SplitMix64(seed ^ 0x504F4F4C, 1 + f*2^32 + block) mod f^2,
 * the same for every batch and head.  f must divide Gh and Gw. */
int area_pool_kv(const area_problem* p, int f, const void* k, const void* v,
                 void* kp, void* vp, void* stream);

/* Phase I cross-scale coarse attention (ai.info summary, Methodology,
 * Phase I): out = softmax(RoPE(q at (y/f, x/f)) kp^T / sqrt(D)) vp for every
 * full-resolution image query (and the T text keys that area_pool_kv puts
 * first).  q: [B][H][T+Gh*Gw][D] bf16 un-rotated; kp, vp as produced by
 * area_pool_kv; out: [B][H][T+Gh*Gw][D] bf16, image rows written.  Workspace:
 * area_workspace_bytes(p, AREA_OP_COARSE). kp and vp are the fp32 rows
 * area_pool_kv produces. */
int area_coarse_attn(const area_problem* p, int f, const void* q, const void* kp,
                     const void* vp, void* out, void* ws, size_t ws_bytes, void* stream);

/* Haar detail map (ai.info summary, Methodology, Phase II: a wavelet map of
 * the hidden state gauges how much fine detail each region holds).
 * latent: [C][Gh][Gw] fp32.  For each
 * 2x2 cell (a b / c d) and channel: LH = (a-b+c-d)/2, HL = (a+b-c-d)/2,
 * HH = (a-b-c+d)/2, summed in float64 as E += (LH^2 + HL^2) + HH^2 in
 * channel order.  energy: [Gh/2][Gw/2] fp32 (E rounded); energy_q:
 * [Gh/2][Gw/2] int32 = min(round_half_even(E * 2^16), 2^31 - 1). */
int area_dwt_detail(const area_problem* p, int C, const float* latent, float* energy,
                    int32_t* energy_q, void* stream);

/* Phase II window plan for step `step` (ai.info summary, Methodology,
 * Phase II; README repository layout: tiling = base tiling, DWT map,
 * splits, Halo, merge weights; bridge = bridge token selection).
 *  energy_q: [Gh/2][Gw/2] int32 from area_dwt_detail (NULL: no splits).
 *  k: [B][H][T+Gh*Gw][D] bf16 un-rotated keys; the bridge is chosen among
 *     the image tokens (NULL or
 *     p->bridge_k == 0: no bridge).
 * Outputs (device):
 *  plan:   area_plan_words(p) int32: header + window records in canonical
 *          order (row-major base windows; a split window replaced in place
 *          by its quadrants TL, TR, BL, BR).  A base window is split when
 *          split_den * S_w * N < split_num * S_tot * |Q_w|, S the integer
 *          sums of energy_q over tokens.  Each record's key rectangle is its
 *          query rectangle dilated by the Halo and clipped to the grid.
 *  wsum:   [Gh*Gw] int32, sum over covering windows of the tent weight
 *          min(u+1, L-u) along y times along x.
 *          The Halo width is p->halo, or, with p->halo_max > 0, drawn per
 *          window from 1..halo_max: 1 + splitmix64(seed ^ 0x48414C4F,
 *          1 + (t * 4096 + parent) * 5 + quadrant + 1) mod halo_max, t the
 *          Phase II step index, parent the base-window index, quadrant -1
 *          for an unsplit window.
 *  bridge_idx: [B][H][R] int32 sorted ascending, R = area_step_info().R of
 *          the step (p->bridge_k, or round(rho w_t)^2): per (b, h), the key
 *          farthest (sum of squared channel deviations, float64, channels in
 *          order) from the exact mean key in each of R cells of the
 *          r_h x r_w grid of area_step_info() (bridge_rh, bridge_rw: the
 *          factor pair of R with the most nearly square cells in tokens,
 *          ties to fewer cell rows; cell (a, c) covers rows
 *          [a Gh / r_h, (a+1) Gh / r_h) and columns [c Gw / r_w,
 *          (c+1) Gw / r_w)); ties to the smaller index.
 * Workspace: area_workspace_bytes(p, AREA_OP_PLAN). */
int area_window_plan(const area_problem* p, int step, const int32_t* energy_q, const void* k,
                     int32_t* plan, int32_t* wsum, int32_t* bridge_idx,
                     void* ws, size_t ws_bytes, void* stream);

/* area_window_plan for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that forbid allocation): the same
 * kernels and outputs, with the plan's scratch in the library's own static
 * device array (16 MiB per GPU, held until the process ends) instead of a
 * workspace argument.  Returns AREA_E_WORKSPACE when
 * area_workspace_bytes(p, AREA_OP_PLAN) exceeds 16 MiB (about B*H*Gh*Gw*D/128
 * bytes with a bridge), AREA_E_HIP if the array cannot be resolved on the
 * current device, else as area_window_plan.  Allocates nothing.  Every call
 * on one GPU uses that GPU's array: calls that may overlap on one GPU
 * (unordered streams) race and must be serialised by the caller. */
int area_window_plan_static(const area_problem* p, int step, const int32_t* energy_q, const void* k,
                            int32_t* plan, int32_t* wsum, int32_t* bridge_idx, void* stream);

/* Phase II windowed attention with blending (ai.info summary, Methodology,
 * Phase II).  For every window of `plan`: its queries attend to the keys of
 * its Halo rectangle plus the bridge tokens outside that rectangle, RoPE at
 * native positions, softmax(q k^T / sqrt(D)) v; each token's output is the
 * tent-weighted average of the outputs of the windows covering it (divided
 * by wsum).  `step` must be the step the plan was built for.  q, k, v:
 * [B][H][T+Gh*Gw][D] bf16 un-rotated; out: same layout, image rows written
 * (each window's key set also holds the T text keys).  bridge_idx may be
 * NULL when the plan has R == 0.  Workspace:
 * area_workspace_bytes(p, AREA_OP_WINDOW). */
int area_window_attn(const area_problem* p, int step, const int32_t* plan, const int32_t* wsum,
                     const int32_t* bridge_idx, const void* q, const void* k, const void* v,
                     void* out, void* ws, size_t ws_bytes, void* stream);

/* Uniform full attention over all Gh*Gw tokens with RoPE at native
 * positions (the baseline of the pages' speedup figures, ai.info summary,
 * Main Findings).  Same layouts as area_window_attn.  Workspace:
 * area_workspace_bytes(p, AREA_OP_FULL). */
int area_full_attn(const area_problem* p, const void* q, const void* k, const void* v,
                   void* out, void* ws, size_t ws_bytes, void* stream);

/* Text queries of a joint sequence (p->T > 0): the T text rows of out get
 * dense attention over all T + Gh*Gw keys with RoPE at native positions
 * (text at (0, 0)) -- the path text queries take in every phase, since only
 * the image keys are pooled or windowed.  Layouts as area_full_attn; only
 * rows 0 .. T-1 of out are written.  Does nothing when p->T == 0.
 * Workspace: area_workspace_bytes(p, AREA_OP_FULL). */
int area_text_attn(const area_problem* p, const void* q, const void* k, const void* v,
                   void* out, void* ws, size_t ws_bytes, void* stream);

/* One attention call of denoising step `step` along the schedule: the
 * pages run Phase I (pooled coarse attention over the pooling ramp) for the
 * first p1_steps denoising steps and Phase II (windowed attention) after
 * that, and keep the original attention when the canvas is at or below the
 * native size (ai.info summary, Methodology, Phase I and Phase II; README,
 * setup note on native resolution).  Dispatches by area_step_info():
 *  AREA_PHASE_FULL:   area_full_attn;
 *  AREA_PHASE_COARSE: area_pool_kv with the step's factor f, then
 *                     area_coarse_attn (and area_text_attn when T > 0);
 *  AREA_PHASE_WINDOW: area_dwt_detail of `latent` (C channels, [C][Gh][Gw]
 *                     fp32; NULL: no quadrant splits), area_window_plan
 *                     (with the bridge when the step has one),
 *                     area_window_attn (and area_text_attn when T > 0).
 * q, k, v: [B][H][T+Gh*Gw][D] bf16 un-rotated; out: same layout.  Every
 * intermediate (pooled K/V, energy map, plan, weight sums, bridge indices)
 * lives in the caller's workspace of area_workspace_bytes(p, AREA_OP_STEP)
 * bytes; nothing is allocated.  Results are identical to calling the
 * individual entry points in that order.  Errors as for those calls; on an
 * error nothing further is enqueued. */
int area_attn_step(const area_problem* p, int step, int C, const float* latent, const void* q,
                   const void* k, const void* v, void* out, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* AREA_H */
