// The pipelined q/k kernel for gfx950 (qk_pipe_kernel) and its launchers:
// per-head RMSNorm + multimodal rotary embedding of token-major q, k (and a
// packed qkv's copied v), one token per wavefront, the token's row-steps as
// one software-pipelined stream.  The arithmetic per element is
// qk_kernel's (mrope_kernels.hip), so the results are bit-identical.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mrope_device.h"

// Resident wavefronts per SIMD the pipelined kernel is compiled for, with
// and without RMSNorm (its registers then fit 512 / this many).  Measured with
// inputs the memory-side cache does not hold and cached row loads: with the
// norm (32 + 4 head bf16 prefill) 3 waves 105.2 us, 4 waves spill (135 us);
// without it (chunked video) 4 waves 32.3 us, 5 waves spill (43.0 us).  A
// spill costs more than its own traffic: scratch loads retire through the
// same in-order counter as the row loads, so each waits for the steps in
// flight.
#ifndef MROPE_PIPE_MIN_WAVES
#define MROPE_PIPE_MIN_WAVES 3
#endif
// Wavefronts per block of the pipelined kernel: one.  A compute unit starts
// a block only where all of its wavefronts fit, so with 4-wavefront blocks a
// slot freed early waits for its block-mates.  Measured from per-wavefront
// timestamps on the 32 + 4 head prefill: 2.63 of 3 wavefronts per SIMD busy
// in the steady state against 2.56 (a freed slot still takes about 1.2 us to
// start its next wavefront), 102.5 -> 101.4 us.
#ifndef MROPE_PIPE_BLOCK_WAVES
#define MROPE_PIPE_BLOCK_WAVES 1
#endif
// Non-temporal row loads (1) or cached ones (0).
#ifndef MROPE_PIPE_NT_LOADS
#define MROPE_PIPE_NT_LOADS 1
#endif
#ifndef MROPE_PIPE_MIN_WAVES_NONORM
#define MROPE_PIPE_MIN_WAVES_NONORM 4
#endif

namespace mrope {

constexpr int kPipeBlockWaves = MROPE_PIPE_BLOCK_WAVES;
constexpr int kPipeBlockThreads = kWaveSize * kPipeBlockWaves;
namespace {

// ---------------------------------------------------------------------------
// The pipelined q/k kernel: cos/sin from positions, one token per wavefront,
// launches of at least one wavefront per token over the whole chip.  The
// token's row-steps -- q's, then k's, then a packed qkv's copied v -- form one
// stream, and the loads of step j + 2 are issued before step j is finished:
// every wavefront keeps two row-steps of loads in flight while it computes.  (In
// qk_kernel a wavefront has loads in flight only while it waits for them, so
// the chip's bytes in flight drop by the share of time its wavefronts spend
// on the norm and the rotation.)  Every row of the wavefront belongs to one
// token, so a lane's cos/sin are the same for all its rows: they are formed
// once (one sincos per lane, exchanged through LDS) and held in registers as
// doubles, which takes the per-step LDS reads and conversions out of the
// loop.  The weights, the token's positions and the first two steps are loaded
// before the sincos.  Every load and store is issued unconditionally -- a
// masked row or a step past the end uses an offset past its buffer -- so the
// compiler's waits on the in-order vector memory counter are exact.  The
// arithmetic per element is qk_kernel's, so the results are bit-identical.
// ---------------------------------------------------------------------------

template <int CB>
struct PipeStep {
  Words<CB> ra, rb;              // the lane's two chunks of its row
  uint32_t you;                  // byte offset of the row's output, or out of range
  int slot;                      // tensor of the step (wave-uniform); kSlots past the end
};

// Position of a wavefront in its step stream.  Wave-uniform: the tensor, the
// steps left in it and its walking constants; per lane: the next row's head
// and byte offsets.
struct PipeCursor {
  int slot, left, H;
  uint32_t xinc, yinc;
  int h;
  uint32_t xo, yo;
};

// Moves the cursor to the first row of the first tensor >= from that has
// steps (n0, n1, n2 for q, k, v), or past the end.  The tensor's fields are
// picked by constant index: a dynamic index into the kernel-argument struct
// would copy it to scratch memory.  One token: row r is head r, at byte
// offset r * D * es of the input and r * head stride of the output.
__device__ __forceinline__ void pipe_enter(PipeCursor& c, const QKParams& p, int from, int n0,
                                           int n1, int n2, int grp, int rpw, int es) {
  int s = from;
  if (s == 0 && n0 == 0) s = 1;
  if (s == 1 && n1 == 0) s = 2;
  if (s == 2 && n2 == 0) s = kSlots;
  c.slot = __builtin_amdgcn_readfirstlane(s);
  if (c.slot >= kSlots) return;
  const int ss = c.slot;
  const int64_t yhs = ss == 0 ? p.y_hs[0] : (ss == 1 ? p.y_hs[1] : p.y_hs[2]);
  c.H = ss == 0 ? p.heads[0] : (ss == 1 ? p.heads[1] : p.heads[2]);
  c.left = ss == 0 ? n0 : (ss == 1 ? n1 : n2);
  c.h = grp;
  c.xo = (uint32_t)((int64_t)grp * p.D * es);
  c.yo = (uint32_t)((int64_t)grp * yhs * es);
  c.xinc = (uint32_t)((int64_t)rpw * p.D * es);
  c.yinc = (uint32_t)((int64_t)rpw * yhs * es);
}

// Issues the loads of the cursor's step into b (masked rows and steps past the
// end load from out of range) and advances the cursor.
template <int CB>
__device__ __forceinline__ void pipe_issue(PipeCursor& c, PipeStep<CB>& b, const QKParams& p,
                                           __amdgpu_buffer_rsrc_t rx0, __amdgpu_buffer_rsrc_t rx1,
                                           __amdgpu_buffer_rsrc_t rx2, int n0, int n1, int n2,
                                           int grp, int rpw, bool lane_on, uint32_t ca,
                                           uint32_t cb, int es) {
  const int s = c.slot;
  const bool have = s < kSlots;
  const bool ok = have && lane_on && c.h < c.H;
  b.slot = s;
  b.you = ok ? c.yo : kOutOfRange;
  const uint32_t xoff = ok ? c.xo : kOutOfRange;
  const __amdgpu_buffer_rsrc_t rx = s == 0 ? rx0 : (s == 1 ? rx1 : rx2);
  // Each input line is read once, by one of a step's two loads: non-temporal.
  // Measured with buffer sets that do not fit the MALL, against cached
  // loads: 32 + 4 head prefill 103.3 -> 101.4 us (100.4 without the norm,
  // from 105.1), Qwen3.5 shape 84.0 -> 81.4 us, chunked video 34.6 -> 33.7
  // us.  Only where the rotation's sets partly stay in the MALL (chunked
  // video over 3 sets, 553 MB) do cached loads win, 32.4 against 33.1 us.
  buf_load<CB, MROPE_PIPE_NT_LOADS>(rx, xoff + ca, b.ra);
  buf_load<CB, MROPE_PIPE_NT_LOADS>(rx, xoff + cb, b.rb);
  if (have) {
    c.xo += c.xinc;
    c.yo += c.yinc;
    c.h += rpw;
    if (--c.left == 0) pipe_enter(c, p, s + 1, n0, n1, n2, grp, rpw, es);
  }
}

// The value of v on lane (lane + HC) for lanes of the first HC of each
// group of 2 * HC lanes (x1 lanes), and on lane (lane - HC) for the others:
// the split-half partner of a rotary chunk in the contiguous-halves layout.
// DPP row shifts stay within 16-lane rows, which hold whole row groups (lpr
// a power of two <= 16).  Every lane of the wavefront executes it.
template <int HC>
__device__ __forceinline__ float xch_partner(float v, bool x2) {
  const int u = __builtin_bit_cast(int, v);
  const int up = __builtin_amdgcn_update_dpp(0, u, 0x100 | HC, 0xF, 0xF, false);  // row_shl
  const int dn = __builtin_amdgcn_update_dpp(0, u, 0x110 | HC, 0xF, 0xF, false);  // row_shr
  return __builtin_bit_cast(float, x2 ? dn : up);
}

// RMSNorm (NORM) and rotation (rot) of one lane's two chunks, with the
// cos/sin of the lane's rotary columns as doubles.  Two layouts: HC == 0, a
// at column col_a and b at its split-half partner (or a second pass-through
// chunk); HC > 0 (partial rotary over at most half the row), a and b at the
// lane's chunk of each half of the row, the rotary chunks on the first 2 * HC
// lanes of a row with the partner of a on the lane HC away (x2 marks the
// second half's lanes).  The arithmetic of finish_steps, element for element.
template <bool BF16, int V, bool NORM, int LPR, int PREC, int HC>
__device__ __forceinline__ void norm_rotate(float (&a)[V], float (&b)[V], const QKParams& p,
                                            int lpr, bool rot, bool x2, const float (&wa)[V],
                                            const float (&wb)[V], const double (&c_)[V],
                                            const double (&s_)[V]) {
  if constexpr (NORM) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      ss = __builtin_fma((double)a[i], (double)a[i], ss);
      ss = __builtin_fma((double)b[i], (double)b[i], ss);
    }
    ss = row_sum<LPR>(ss, lpr);
    const float rs = rsqrt_to_f32(ss * p.inv_d + (double)p.eps);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      a[i] = a[i] * rs;
      b[i] = b[i] * rs;
    }
    if constexpr (BF16) round_bf16_chunks<V>(a, b);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      a[i] = a[i] * wa[i];
      b[i] = b[i] * wb[i];
    }
    if constexpr (BF16) round_bf16_chunks<V>(a, b);
  }
  if constexpr (HC > 0) {
    float pa[V];
#pragma unroll
    for (int i = 0; i < V; ++i) pa[i] = xch_partner<HC>(a[i], x2);
    if (rot) {
      // x1 lanes: x1 * cos - x2 * sin; x2 lanes: x2 * cos + x1 * sin.
      if constexpr (PREC == MROPE_PRECISION_EXACT) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const double ps = (double)pa[i] * s_[i];
          a[i] = (float)__builtin_fma((double)a[i], c_[i], x2 ? ps : -ps);
        }
      } else {
#pragma clang fp contract(off)
#pragma unroll
        for (int i = 0; i < V; ++i) {
          float c1 = (float)c_[i], s1 = (float)s_[i];
          if constexpr (BF16 && PREC == MROPE_PRECISION_DTYPE) {
            c1 = round_bf16(c1);
            s1 = round_bf16(s1);
          }
          float p1 = a[i] * c1;
          float p2 = pa[i] * s1;
          if constexpr (BF16 && PREC == MROPE_PRECISION_DTYPE) {
            p1 = round_bf16(p1);
            p2 = round_bf16(p2);
          }
          a[i] = x2 ? p1 + p2 : p1 - p2;
        }
      }
    }
  } else if (rot) {
    if constexpr (PREC == MROPE_PRECISION_EXACT) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const double y1 = a[i];
        const double y2 = b[i];
        const double o1 = __builtin_fma(y1, c_[i], -(y2 * s_[i]));
        const double o2 = __builtin_fma(y2, c_[i], y1 * s_[i]);
        a[i] = (float)o1;
        b[i] = (float)o2;
      }
    } else {
      rotate_tensor_ops<BF16 && PREC == MROPE_PRECISION_DTYPE, V>(a, b, c_, s_, c_, s_);
    }
  }
}

// Finishes a step: RMSNorm and rotation of q and k rows (v rows are copied)
// and the two stores.  A step past the end (valid false) skips the
// arithmetic; its stores, like those of masked rows, are out of range.
template <bool BF16, int V, bool NORM, int LPR, int PREC, int HC>
__device__ __forceinline__ void pipe_finish(const PipeStep<(BF16 ? 2 : 4) * V>& b, bool valid,
                                            const QKParams& p, int lpr, bool rot, bool x2,
                                            uint32_t ca,
                                            uint32_t cb, const double (&c_)[V],
                                            const double (&s_)[V], const float (&wqa)[V],
                                            const float (&wqb)[V], const float (&wka)[V],
                                            const float (&wkb)[V], __amdgpu_buffer_rsrc_t ry0,
                                            __amdgpu_buffer_rsrc_t ry1,
                                            __amdgpu_buffer_rsrc_t ry2) {
  constexpr int CB = (BF16 ? 2 : 4) * V;
  Words<CB> oa = b.ra, ob = b.rb;
  if (valid && b.slot < 2) {
    float a[V], c[V];
    unpack<BF16, V>(b.ra, a);
    unpack<BF16, V>(b.rb, c);
    if (b.slot == 0)
      norm_rotate<BF16, V, NORM, LPR, PREC, HC>(a, c, p, lpr, rot, x2, wqa, wqb, c_, s_);
    else
      norm_rotate<BF16, V, NORM, LPR, PREC, HC>(a, c, p, lpr, rot, x2, wka, wkb, c_, s_);
    pack<BF16, V>(a, oa);
    pack<BF16, V>(c, ob);
  }
  const __amdgpu_buffer_rsrc_t ry = b.slot == 0 ? ry0 : (b.slot == 1 ? ry1 : ry2);
  buf_store<BF16, CB>(ry, b.you + ca, oa);
  buf_store<BF16, CB>(ry, b.you + cb, ob);
}

template <bool BF16, int V, bool NORM, int LPR, int PREC, int HC>
__global__ void __launch_bounds__(kPipeBlockThreads)
__attribute__((amdgpu_waves_per_eu(NORM ? MROPE_PIPE_MIN_WAVES : MROPE_PIPE_MIN_WAVES_NONORM)))
qk_pipe_kernel(const QKParams p, const ColTable tab) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int CB = ES * V;
  extern __shared__ double lds[];
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int half = p.half;
  float* lc = reinterpret_cast<float*>(lds) + wib * (2 * half);
  float* ls = lc + half;

  const int lpr = LPR > 0 ? LPR : p.lpr;
  const int rpw = LPR > 0 ? kWaveSize / (LPR > 0 ? LPR : 1) : p.rpw;
  const int grp = lane / lpr;
  const int l = lane - grp * lpr;
  const bool lane_on = grp < rpw;
  // The lane's two chunks (columns col_a and col_b) and the column of its
  // cos/sin (cj).  HC == 0: col_a rotary or pass-through, col_b its split-half
  // partner or a second pass-through chunk.  HC > 0 (HC == lrot, partial
  // rotary over at most half the row): one chunk in each half of the row, so
  // each store instruction writes whole cache lines; the rotary chunks are
  // the first 2 * HC of the row, x1 on lanes l < HC and x2 on the next HC.
  bool rot, x2 = false;
  int col_a, col_b, cj;
  if constexpr (HC > 0) {
    col_a = l * V;
    col_b = (lpr + l) * V;
    rot = l < 2 * HC;
    x2 = l >= HC;
    cj = rot ? (x2 ? l - HC : l) * V : 0;
  } else {
    rot = l < p.lrot;
    if (l < p.lrot) {
      col_a = l * V;
      col_b = half + l * V;
    } else {
      const int m = l - p.lrot;
      const int npass = lpr - p.lrot;
      col_a = p.rd + m * V;
      col_b = p.rd + (npass + m) * V;
    }
    cj = rot ? col_a : 0;
  }
  const uint32_t ca = (uint32_t)(col_a * ES);
  const uint32_t cb = (uint32_t)(col_b * ES);

  const int64_t t0 = (int64_t)blockIdx.x * kPipeBlockWaves + wib;
  if (t0 >= p.T) return;
  // Row-steps of each tensor (wave-uniform scalars: no private arrays, so
  // the buffer descriptors chosen from them stay in scalar registers).
  const int n0 = (p.heads[0] + rpw - 1) / rpw;
  const int n1 = (p.heads[1] + rpw - 1) / rpw;
  const int n2 = (p.heads[2] + rpw - 1) / rpw;
  const int N = n0 + n1 + n2;
  if (N == 0) return;

  // The token's rows of each tensor (32-bit byte offsets inside them).
#define MROPE_X_RSRC(s)                                                          \
  buffer_of(static_cast<const char*>(p.x[s]) + t0 * p.x_ts[s] * ES,              \
            (uint32_t)((int64_t)p.heads[s] * p.D * ES))
#define MROPE_Y_RSRC(s)                                                          \
  buffer_of(static_cast<const char*>(p.y[s]) + t0 * p.y_ts[s] * ES,              \
            p.heads[s] > 0 ? (uint32_t)(((int64_t)(p.heads[s] - 1) * p.y_hs[s] + p.D) * ES) : 0u)
  const __amdgpu_buffer_rsrc_t rx0 = MROPE_X_RSRC(0), rx1 = MROPE_X_RSRC(1), rx2 = MROPE_X_RSRC(2);
  const __amdgpu_buffer_rsrc_t ry0 = MROPE_Y_RSRC(0), ry1 = MROPE_Y_RSRC(1), ry2 = MROPE_Y_RSRC(2);
#undef MROPE_X_RSRC
#undef MROPE_Y_RSRC

  // 1. RMSNorm weights of q and k (tiny, shared by every wavefront).
  Words<CB> wq_a = {}, wq_b = {}, wk_a = {}, wk_b = {};
  if constexpr (NORM) {
    const __amdgpu_buffer_rsrc_t rq =
        buffer_of(p.w[0], p.heads[0] > 0 ? (uint32_t)(p.D * ES) : 0u);
    const __amdgpu_buffer_rsrc_t rk =
        buffer_of(p.w[1], p.heads[1] > 0 ? (uint32_t)(p.D * ES) : 0u);
    buf_load<CB>(rq, ca, wq_a);
    buf_load<CB>(rq, cb, wq_b);
    buf_load<CB>(rk, ca, wk_a);
    buf_load<CB>(rk, cb, wk_b);
  }

  // 2. What the sincos of the token's first 2 x 64 columns need: positions
  // (the axis from the fitted rule, no table load) and inv_freq.
  constexpr int kPrePos = 2;
  int32_t pos_pre[kPrePos];
  float inv_pre[kPrePos];
#pragma unroll
  for (int m = 0; m < kPrePos; ++m) {
    const int idx = lane + m * kWaveSize;
    const int j = idx < half ? idx : 0;
    int ax;
    if (p.ax_mode == 0) ax = (j >= p.ax_a) + (j >= p.ax_b);
    else if (p.ax_mode == 1) ax = (j % 3 == 1 && j < p.ax_a) ? 1 : (j % 3 == 2 && j < p.ax_b) ? 2 : 0;
    else ax = tab.axis[j];
    pos_pre[m] = p.pos[(int64_t)ax * p.pos_stride + t0];
    inv_pre[m] = tab.inv[j];
  }

  // 3. The step stream, and the loads of its first two steps.
  PipeCursor cur;
  pipe_enter(cur, p, 0, n0, n1, n2, grp, rpw, ES);
#define MROPE_ISSUE(b) \
  pipe_issue<CB>(cur, b, p, rx0, rx1, rx2, n0, n1, n2, grp, rpw, lane_on, ca, cb, ES)
  // The step buffers rotate through the unrolled loop bodies below.
  PipeStep<CB> b0, b1, b2;
  MROPE_ISSUE(b0);
  MROPE_ISSUE(b1);

  // 4. The token's cos/sin, one column per lane, exchanged through the
  // wavefront's LDS slice while the first two steps load.
#pragma unroll
  for (int m = 0; m < kPrePos; ++m) {
    const int j = lane + m * kWaveSize;
    if (j < half) {
      const int32_t pp = pos_pre[m];
      float c, s;
      if (p.cs_cache != nullptr && (uint32_t)pp < (uint32_t)p.cache_rows) {
        cached_cos_sin(p.cs_cache, (int64_t)pp * p.n_freq + tab.fidx[j], c, s);
      } else {
        angle_cos_sin(pp, inv_pre[m], c, s);
      }
      lc[j] = c;
      ls[j] = s;
    }
  }
  for (int j = lane + kPrePos * kWaveSize; j < half; j += kWaveSize) {
    const int32_t pp = p.pos[(int64_t)tab.axis[j] * p.pos_stride + t0];
    float c, s;
    if (p.cs_cache != nullptr && (uint32_t)pp < (uint32_t)p.cache_rows) {
      cached_cos_sin(p.cs_cache, (int64_t)pp * p.n_freq + tab.fidx[j], c, s);
    } else {
      angle_cos_sin(pp, tab.inv[j], c, s);
    }
    lc[j] = c;
    ls[j] = s;
  }
  // LDS traffic of one wavefront is processed in order; this only keeps the
  // compiler from moving the reads above the writes.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // This lane's columns (pass-through lanes read column 0: unused)
  double c_[V], s_[V];
  {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      c_[i] = (double)lc[cj + i];
      s_[i] = (double)ls[cj + i];
    }
  }

  float wqa[V], wqb[V], wka[V], wkb[V];
  unpack<BF16, V>(wq_a, wqa);
  unpack<BF16, V>(wq_b, wqb);
  unpack<BF16, V>(wk_a, wka);
  unpack<BF16, V>(wk_b, wkb);

  // 5. Finish step j while steps j + 1 and j + 2 load.
#define MROPE_FINISH(b, valid)                                                                  \
  pipe_finish<BF16, V, NORM, LPR, PREC, HC>(b, valid, p, lpr, rot, x2, ca, cb, c_, s_, wqa, wqb, \
                                            wka, wkb, ry0, ry1, ry2)
  for (int j = 0; j < N; j += 3) {
    MROPE_ISSUE(b2);
    MROPE_FINISH(b0, j < N);
    MROPE_ISSUE(b0);
    MROPE_FINISH(b1, j + 1 < N);
    MROPE_ISSUE(b1);
    MROPE_FINISH(b2, j + 2 < N);
  }
#undef MROPE_ISSUE
#undef MROPE_FINISH
}

template <bool BF16, int V, bool NORM, int LPR, int PREC, int HC>
int launch_pipe_t(QKParams p, const ColTable& tab, hipStream_t st) {
  fit_axis_rule(tab, p.half, p);
  p.nt = 1;
  p.parts = 1;
  const int64_t blocks = (p.T + kPipeBlockWaves - 1) / kPipeBlockWaves;
  int lds = kPipeBlockWaves * 2 * p.half * (int)sizeof(float);
  if (p.waves_cap > 0) {
    // waves_cap wavefronts per SIMD = 4 * waves_cap per compute unit
    const int cap_lds = (kLdsPerCu * kPipeBlockWaves / (4 * p.waves_cap)) & ~511;
    if (cap_lds > lds) lds = cap_lds;
  }
  hipLaunchKernelGGL((qk_pipe_kernel<BF16, V, NORM, LPR, PREC, HC>), dim3((unsigned)blocks),
                     dim3(kPipeBlockThreads), lds, st, p, tab);
  return (int)hipGetLastError();
}

// The contiguous-halves layout (HC = rotary chunks per half) serves bf16 rows
// of 8 or 16 lanes whose rotary columns fit in the first half of the row:
// partial rotary, where the split-half layout writes two cache lines of each
// row half from each of the two store instructions.  Measured on the Qwen3.5
// shape (256-wide heads, 64 rotary columns), rotating buffer sets, cached row
// loads: 85.4 -> 83.5 us.
template <bool BF16, int V, bool NORM, int LPR, int PREC>
int launch_pipe_hc(const QKParams& p, const ColTable& tab, hipStream_t st) {
  if constexpr (BF16 && LPR >= 8) {
    if (p.rd < p.D && 2 * p.lrot <= LPR) {
      switch (p.lrot) {
        case 2: return launch_pipe_t<BF16, V, NORM, LPR, PREC, 2>(p, tab, st);
        case 4: return launch_pipe_t<BF16, V, NORM, LPR, PREC, 4>(p, tab, st);
        case 8:
          if constexpr (LPR == 16) return launch_pipe_t<BF16, V, NORM, LPR, PREC, 8>(p, tab, st);
          break;
      }
    }
  }
  return launch_pipe_t<BF16, V, NORM, LPR, PREC, 0>(p, tab, st);
}

template <bool BF16, int V, bool NORM, int LPR>
int launch_pipe_prec(int prec, const QKParams& p, const ColTable& tab, hipStream_t st) {
  switch (prec) {
    case MROPE_PRECISION_EXACT:
      return launch_pipe_hc<BF16, V, NORM, LPR, MROPE_PRECISION_EXACT>(p, tab, st);
    case MROPE_PRECISION_DTYPE:
      return launch_pipe_hc<BF16, V, NORM, LPR, MROPE_PRECISION_DTYPE>(p, tab, st);
    case MROPE_PRECISION_FP32:
      if constexpr (BF16)
        return launch_pipe_hc<BF16, V, NORM, LPR, MROPE_PRECISION_FP32>(p, tab, st);
      break;
  }
  return (int)hipErrorInvalidValue;
}

template <bool BF16, int V, bool NORM>
int launch_pipe_lpr(int prec, const QKParams& p, const ColTable& tab, hipStream_t st) {
  switch (p.lpr) {
    case 8: return launch_pipe_prec<BF16, V, NORM, 8>(prec, p, tab, st);
    case 16: return launch_pipe_prec<BF16, V, NORM, 16>(prec, p, tab, st);
  }
  return launch_pipe_prec<BF16, V, NORM, 0>(prec, p, tab, st);
}

}  // namespace

int launch_qk_pipe(int dtype, int vec, bool norm, int prec, const QKParams& p,
                   const ColTable& tab, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == MROPE_DTYPE_BF16 && vec == 8)
    return norm ? launch_pipe_lpr<true, 8, true>(prec, p, tab, st)
                : launch_pipe_lpr<true, 8, false>(prec, p, tab, st);
  if (dtype == MROPE_DTYPE_F32 && vec == 4)
    return norm ? launch_pipe_lpr<false, 4, true>(prec, p, tab, st)
                : launch_pipe_lpr<false, 4, false>(prec, p, tab, st);
  return (int)hipErrorInvalidValue;
}

}  // namespace mrope
