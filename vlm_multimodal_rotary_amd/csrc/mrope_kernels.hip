// HIP kernels for gfx950: per-head RMSNorm + multimodal rotary embedding over
// token-major q[T][hq][D] and k[T][hk][D].
//
// The path is elementwise and HBM-bound (about 7 flops per element), so there
// is no MFMA here.  The design points:
//
//  * A head row of D elements is covered by lpr = D / (2V) adjacent lanes,
//    each owning two V-element chunks (16 bytes for bf16 V = 8 or fp32
//    V = 4).  A rotary lane owns the chunk at column c and the one at c + h
//    (h = rotary_dim / 2), so the split-half rotation of the RoPE post's
//    rotate_half / apply_rotary_pos_emb needs no cross-lane exchange.  Lanes
//    past the rotary lanes own pass-through chunks (partial rotary).
//  * One wavefront handles a tile of nt consecutive tokens.  It first forms
//    cos/sin for every (token, column < h) of the tile once, one sincos per
//    lane with no redundancy, into its own LDS slice; every q and k head of a
//    token then reuses them (the pages compute cos/sin once per forward and
//    share them over heads).  Rows of the tile are walked with 64/lpr rows per
//    instruction and U rows in flight per lane.  With RMSNorm (and in decode)
//    the first row-steps are loaded before the sincos and finished after it,
//    so that the sincos overlaps their memory latency.
//  * flat_kernel (rows that are not whole 256-byte line pairs) and
//    stage_kernel (bf16 per-head planes, through LDS) serve the positions
//    path without RMSNorm, and qk_pipe_kernel (mrope_pipe.hip) the positions
//    path of launches of 2048 tokens or more with 16-byte chunks; the host
//    picks the kernel by shape.  Helpers shared with mrope_pipe.hip are in
//    mrope_device.h.
//  * The RMS reduction of a row runs over its lpr lanes with DPP
//    (quad_perm, row_half_mirror, row_mirror) on float64 partial sums.
//  * Numerics follow the pages' conventions with the rounding points made
//    exact: the angle is the binary32 product float(p) * inv_freq; cos/sin
//    are evaluated in double and rounded once to binary32; the sum of squares
//    is accumulated in double; r = fl32(1/sqrt(mean + eps)); the normalised
//    value is cast to the input dtype before the weight multiply and again
//    after it; the rotation is evaluated in double from the stored values and
//    the binary32 cos/sin (both products are exact) and rounded once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mrope_device.h"

// Row-steps whose loads are issued together, per lane, by element type.
#ifndef MROPE_ROWS_IN_FLIGHT_BF16
#define MROPE_ROWS_IN_FLIGHT_BF16 2
#endif
#ifndef MROPE_ROWS_IN_FLIGHT_F32
#define MROPE_ROWS_IN_FLIGHT_F32 4
#endif
// Row-steps in flight for chunks narrower than 16 bytes (e.g. bf16 with a
// half head of 36: 8-byte chunks).
#ifndef MROPE_ROWS_IN_FLIGHT_NARROW
#define MROPE_ROWS_IN_FLIGHT_NARROW 2
#endif
// Wavefronts a launch aims to have in flight before it splits tiles.
#ifndef MROPE_MIN_WAVES
#define MROPE_MIN_WAVES 2048
#endif

namespace mrope {
namespace {

constexpr int64_t kMinWaves = MROPE_MIN_WAVES;

// Per-tensor state of one tile while its rows are processed.
template <int CB>
struct SlotState {
  __amdgpu_buffer_rsrc_t rx, ry;  // tile-local buffers of input and output
  uint32_t xo, yo;                // byte offsets of this lane's next row
  uint32_t xinc, yinc;            // advance by rpw rows ...
  uint32_t xwrap, ywrap;          // ... plus this when the head index wraps
  int tl, h;                      // token (in tile) and head of the next row
  int dq, dr;                     // rpw = dq * H + dr
  int H, nrows;
};

template <int CB, int UU>
struct StepLoads {
  Words<CB> ra[UU], rb[UU];
  int tlu[UU];
  bool ok[UU];
  uint32_t you[UU];
};

template <int CB, int UU>
__device__ __forceinline__ void load_steps(SlotState<CB>& st, int r0, int grp, int rpw,
                                           bool lane_on, uint32_t ca, uint32_t cb,
                                           StepLoads<CB, UU>& L) {
#pragma unroll
  for (int u = 0; u < UU; ++u) {
    const int r = r0 + u * rpw + grp;
    L.ok[u] = lane_on && r < st.nrows;
    L.tlu[u] = st.tl;
    L.you[u] = L.ok[u] ? st.yo : kOutOfRange;
    const uint32_t xoff = L.ok[u] ? st.xo : kOutOfRange;
    buf_load<CB>(st.rx, xoff + ca, L.ra[u]);
    buf_load<CB>(st.rx, xoff + cb, L.rb[u]);
    st.xo += st.xinc;
    st.yo += st.yinc;
    st.h += st.dr;
    st.tl += st.dq;
    if (st.h >= st.H) {
      st.h -= st.H;
      ++st.tl;
      st.xo += st.xwrap;
      st.yo += st.ywrap;
    }
  }
}

template <bool BF16, int V, int CS, bool NORM, int LPR, int PREC, int UU, typename CsT>
__device__ __forceinline__ void finish_steps(const SlotState<(BF16 ? 2 : 4) * V>& st,
                                             const StepLoads<(BF16 ? 2 : 4) * V, UU>& L,
                                             const QKParams& p, int lpr, bool rot, uint32_t ca,
                                             uint32_t cb, int col_a, const float (&wa)[V],
                                             const float (&wb)[V], const CsT* lc,
                                             const CsT* ls, int64_t t0) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int CB = ES * V;
  const Words<CB>(&ra)[UU] = L.ra;
  const Words<CB>(&rb)[UU] = L.rb;
  const int(&tlu)[UU] = L.tlu;
  const bool(&ok)[UU] = L.ok;
  const uint32_t(&you)[UU] = L.you;
#pragma unroll
  for (int u = 0; u < UU; ++u) {
    if constexpr (CS == kCsNone && !NORM) {
      // plain copy: the loaded words go back out unchanged
      buf_store<BF16, CB>(st.ry, you[u] + ca, ra[u]);
      buf_store<BF16, CB>(st.ry, you[u] + cb, rb[u]);
      continue;
    }
    float a[V], b[V];
    unpack<BF16, V>(ra[u], a);
    unpack<BF16, V>(rb[u], b);

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

    if constexpr (CS != kCsNone) {
      if (rot) {
        // Rows past the tile's end read the cos/sin of the tile's first
        // token, so every read stays inside the LDS slice / caller tables.
        const int tlr = ok[u] ? tlu[u] : 0;
        double ca_[V], sa_[V], cb_[V], sb_[V];
        if constexpr (CS == kCsFromPositions || CS == kCsDecode) {
          const int o = tlr * p.half + col_a;
#pragma unroll
          for (int i = 0; i < V; ++i) {
            ca_[i] = (double)lc[o + i];
            sa_[i] = (double)ls[o + i];
            cb_[i] = ca_[i];
            sb_[i] = sa_[i];
          }
        } else {
          const int64_t o = (t0 + tlr) * p.cs_ts + col_a;
          const int64_t ob = o - col_a + (int64_t)(cb / ES);
#pragma unroll
          for (int i = 0; i < V; ++i) {
            ca_[i] = (double)p.cos[o + i];
            sa_[i] = (double)p.sin[o + i];
            cb_[i] = (double)p.cos[ob + i];
            sb_[i] = (double)p.sin[ob + i];
          }
        }
        if constexpr (PREC == MROPE_PRECISION_EXACT) {
#pragma unroll
          for (int i = 0; i < V; ++i) {
            const double y1 = a[i];
            const double y2 = b[i];
            const double o1 = __builtin_fma(y1, ca_[i], -(y2 * sa_[i]));
            const double o2 = __builtin_fma(y2, cb_[i], y1 * sb_[i]);
            a[i] = (float)o1;
            b[i] = (float)o2;
          }
        } else {
          rotate_tensor_ops<BF16 && PREC == MROPE_PRECISION_DTYPE, V>(a, b, ca_, sa_, cb_, sb_);
        }
      }
    }

    Words<CB> wa_out, wb_out;
    pack<BF16, V>(a, wa_out);
    pack<BF16, V>(b, wb_out);
    buf_store<BF16, CB>(st.ry, you[u] + ca, wa_out);
    buf_store<BF16, CB>(st.ry, you[u] + cb, wb_out);
  }
}

template <bool BF16, int V, int CS, bool NORM, int LPR, int PREC, int UU, typename CsT>
__device__ __forceinline__ void process_steps(SlotState<(BF16 ? 2 : 4) * V>& st, int r0,
                                              const QKParams& p, int grp, int rpw, int lpr,
                                              bool lane_on, bool rot, uint32_t ca, uint32_t cb,
                                              int col_a, const float (&wa)[V],
                                              const float (&wb)[V], const CsT* lc,
                                              const CsT* ls, int64_t t0) {
  StepLoads<(BF16 ? 2 : 4) * V, UU> L;
  load_steps<(BF16 ? 2 : 4) * V, UU>(st, r0, grp, rpw, lane_on, ca, cb, L);
  finish_steps<BF16, V, CS, NORM, LPR, PREC, UU>(st, L, p, lpr, rot, ca, cb, col_a, wa, wb, lc, ls,
                                                t0);
}

// Wavefront w owns part w % parts of the tile of tokens [t0, t0 + nt),
// t0 = (w / parts) * nt (parts = 1 on large launches): first the tile's
// cos/sin (in its LDS slice), then its part of the tile's row-steps -- q, k
// and a packed qkv's copied v, in that order -- U per batch of loads.
// Wavefronts are short-lived and many; the hardware overlaps them, and the
// chip's active window of rows stays contiguous.
template <bool BF16, int V, int CS, bool NORM, int LPR, int PREC>
__global__ void __launch_bounds__(kBlockThreads)
qk_kernel(const QKParams p, const ColTable tab) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int CB = ES * V;
  constexpr int U = CB < 16 ? MROPE_ROWS_IN_FLIGHT_NARROW
                            : (BF16 ? MROPE_ROWS_IN_FLIGHT_BF16 : MROPE_ROWS_IN_FLIGHT_F32);
  // cos/sin are binary32 values: LDS holds them as float (half the bytes of
  // double; measured 0.9% faster on the headline, 1.4% on chunked video) and
  // the rotation widens them exactly.
  typedef float cs_t;
  extern __shared__ double lds[];

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int half = p.half;
  cs_t* lc = reinterpret_cast<cs_t*>(lds) + wib * (2 * p.nt * half);
  cs_t* ls = lc + p.nt * half;

  const int lpr = LPR > 0 ? LPR : p.lpr;
  const int rpw = LPR > 0 ? kWaveSize / (LPR > 0 ? LPR : 1) : p.rpw;
  const int grp = lane / lpr;
  const int l = lane - grp * lpr;
  const bool lane_on = grp < rpw;
  const bool rot = (CS != kCsNone) && (l < p.lrot);
  int col_a, col_b;
  if (l < p.lrot) {
    col_a = l * V;
    col_b = half + l * V;
  } else {
    const int m = l - p.lrot;
    const int npass = lpr - p.lrot;
    col_a = p.rd + m * V;
    col_b = p.rd + (npass + m) * V;
  }
  const uint32_t ca = (uint32_t)(col_a * ES);
  const uint32_t cb = (uint32_t)(col_b * ES);

  // This wavefront's tile (tokens [t0, t0 + ntok)) and its part of the
  // tile's row-steps (q steps, then k steps, then v steps), p.parts parts per
  // tile.
  const uint32_t wave = blockIdx.x * (uint32_t)kWavesPerBlock + (uint32_t)wib;
  // Large launches have one part per tile; the divisions are skipped there.
  const bool split = p.parts > 1;
  const uint32_t tile = split ? wave / (uint32_t)p.parts : wave;
  const int part = split ? (int)(wave - tile * (uint32_t)p.parts) : 0;
  const int64_t t0 = (int64_t)tile * p.nt;
  if (t0 >= p.T) return;
  const int ntok = (int)((p.T - t0) < p.nt ? (p.T - t0) : p.nt);
  int pre[kSlots + 1];   // first step of each tensor
  pre[0] = 0;
#pragma unroll
  for (int s = 0; s < kSlots; ++s) pre[s + 1] = pre[s] + (ntok * p.heads[s] + rpw - 1) / rpw;
  const int steps_all = pre[kSlots];
  const int step_begin = split ? steps_all * part / p.parts : 0;
  const int step_end = split ? steps_all * (part + 1) / p.parts : steps_all;
  // Walking state of tensor s from step lo on.
  auto make_state = [&](int s, int lo) {
    const int H = p.heads[s];
    const int64_t xts = p.x_ts[s];
    const int64_t yts = p.y_ts[s];
    const int64_t yhs = p.y_hs[s];
    SlotState<CB> st;
    // Tile-local buffers: byte offsets below stay within 32 bits.
    st.rx = buffer_of(static_cast<const char*>(p.x[s]) + t0 * xts * ES,
                      (uint32_t)(((int64_t)(ntok - 1) * xts + (int64_t)H * p.D) * ES));
    st.ry = buffer_of(static_cast<const char*>(p.y[s]) + t0 * yts * ES,
                      (uint32_t)(((int64_t)(ntok - 1) * yts + (int64_t)(H - 1) * yhs + p.D) * ES));
    st.H = H;
    st.nrows = ntok * H;
    st.dq = p.dq[s];
    st.dr = p.dr[s];
    // First row of this lane: r = lo * rpw + grp; r / H through a binary32
    // reciprocal (r < 2^23, so the estimate is off by at most one), corrected.
    const int r_first = lo * rpw + grp;
    st.tl = (int)((float)r_first * p.inv_heads[s]);
    if (st.tl * H > r_first) --st.tl;
    if ((st.tl + 1) * H <= r_first) ++st.tl;
    st.h = r_first - st.tl * H;
    st.xo = (uint32_t)(((int64_t)st.tl * xts + (int64_t)st.h * p.D) * ES);
    st.yo = (uint32_t)(((int64_t)st.tl * yts + (int64_t)st.h * yhs) * ES);
    st.xinc = (uint32_t)(((int64_t)st.dq * xts + (int64_t)st.dr * p.D) * ES);
    st.yinc = (uint32_t)(((int64_t)st.dq * yts + (int64_t)st.dr * yhs) * ES);
    st.xwrap = (uint32_t)((xts - (int64_t)H * p.D) * ES);
    st.ywrap = (uint32_t)((yts - (int64_t)H * yhs) * ES);
    return st;
  };
  // Decode: rotated k goes to its cache row; a row outside [0, capacity) gets
  // an empty buffer, so its stores are dropped.
  auto k_cache_buffer = [&](int64_t seq, int32_t slot) {
    const bool in_cache = slot >= 0 && slot < p.kc_cap;
    return buffer_of(static_cast<const char*>(p.y[1]) +
                         (seq * p.kc_seq + (int64_t)(in_cache ? slot : 0) * p.kc_tok) * ES,
                     in_cache ? (uint32_t)((int64_t)p.heads[1] * p.D * ES) : 0u);
  };
  // Decode and the fused RMSNorm path: the part's first row-steps (and their
  // norm weights) are loaded before the tile's cos/sin are formed, and
  // finished right after, so the sincos overlaps their memory latency.
  // Decode preloads one step, the positions path two (three or four measured
  // slower: more registers, or no gain).  Vector memory waits count loads in
  // issue order, so what the cos/sin needs (inv_freq values, and on the
  // positions path the positions, addressed through the axis rule rather
  // than a table load) is loaded first, and the row loads are issued on
  // every path (out of range where there is no work): the cos/sin then waits
  // for its own inputs alone.
  [[maybe_unused]] int s_pre = -1;
  [[maybe_unused]] SlotState<CB> st_pre;
  constexpr int kPreSteps = 2;   // row-steps preloaded on the positions path (decode: 1)
  [[maybe_unused]] StepLoads<CB, 1> L_pre, L_more[kPreSteps - 1];
  [[maybe_unused]] int n_pre_steps = 0;
  [[maybe_unused]] float inv_first = 0.f;
  [[maybe_unused]] Words<CB> w_pre_a, w_pre_b;
  // Positions path: the cos/sin inputs of the prologue's first kPrePos
  // iterations (tiles up to 128 (token, column) pairs) are loaded up front.
  // Without RMSNorm the preload measured no faster, so it is off there.
  constexpr int kPrePos = 2;
  constexpr bool kPrePosPath = CS == kCsFromPositions && NORM;
  [[maybe_unused]] int32_t pos_pre[kPrePos];
  [[maybe_unused]] float inv_pre[kPrePos];
  if constexpr (kPrePosPath) {
    const int n_cs = ntok * half;
#pragma unroll
    for (int m = 0; m < kPrePos; ++m) {
      const int idx = lane + m * kWaveSize;
      const int id = idx < n_cs ? idx : 0;
      const int tl = id / half;
      const int j = id - tl * half;
      int ax;
      if (p.ax_mode == 0) ax = (j >= p.ax_a) + (j >= p.ax_b);
      else if (p.ax_mode == 1) ax = (j % 3 == 1 && j < p.ax_a) ? 1 : (j % 3 == 2 && j < p.ax_b) ? 2 : 0;
      else ax = tab.axis[j];
      pos_pre[m] = p.pos[(int64_t)ax * p.pos_stride + t0 + tl];
      inv_pre[m] = tab.inv[j];
    }
  }
  if constexpr (CS == kCsDecode || kPrePosPath) {
    if constexpr (CS == kCsDecode) {
      if (lane < half) inv_first = tab.inv[lane];
    }
    const int lo0 = (step_begin > pre[0] ? step_begin : pre[0]) - pre[0];
    const int hi0 = (step_end < pre[1] ? step_end : pre[1]) - pre[0];
    const int lo1 = (step_begin > pre[1] ? step_begin : pre[1]) - pre[1];
    const int hi1 = (step_end < pre[2] ? step_end : pre[2]) - pre[1];
    int lo_pre = 0;
    if (p.heads[0] > 0 && lo0 < hi0) {
      s_pre = 0;
      lo_pre = lo0;
    } else if (p.heads[1] > 0 && lo1 < hi1) {
      s_pre = 1;
      lo_pre = lo1;
    }
    st_pre = make_state(s_pre >= 0 ? s_pre : 0, lo_pre);
    if constexpr (NORM) {
      const __amdgpu_buffer_rsrc_t rw =
          buffer_of(p.w[s_pre >= 0 ? s_pre : 0], s_pre >= 0 ? (uint32_t)(p.D * ES) : 0u);
      buf_load<CB>(rw, ca, w_pre_a);
      buf_load<CB>(rw, cb, w_pre_b);
    }
    load_steps<CB, 1>(st_pre, lo_pre * rpw, grp, rpw, lane_on && s_pre >= 0, ca, cb, L_pre);
    if constexpr (kPrePosPath) {
      const int hi_pre = s_pre == 0 ? hi0 : hi1;
      const int avail = s_pre < 0 ? 0 : hi_pre - lo_pre;
      n_pre_steps = avail < kPreSteps ? avail : kPreSteps;
#pragma unroll
      for (int u = 0; u < kPreSteps - 1; ++u)
        load_steps<CB, 1>(st_pre, (lo_pre + 1 + u) * rpw, grp, rpw, lane_on && u + 1 < n_pre_steps,
                          ca, cb, L_more[u]);
    } else {
      n_pre_steps = s_pre >= 0 ? 1 : 0;
    }
  }
  {
    // Decode: token t0 is token i of sequence b; its text position (the same
    // on every axis) continues the sequence's cache.
    [[maybe_unused]] int32_t dec_slot = 0;
    [[maybe_unused]] int64_t dec_seq = 0;
    if constexpr (CS == kCsDecode) {
      dec_seq = t0 / p.new_tokens;
      const int i = (int)(t0 - dec_seq * p.new_tokens);
      dec_slot = p.cache_len[dec_seq] + i;
      const int32_t pp = dec_slot + (p.rope_delta != nullptr ? p.rope_delta[dec_seq] : 0);
      if (lane < half) {
        float c, s;
        angle_cos_sin(pp, inv_first, c, s);
        lc[lane] = (cs_t)c;
        ls[lane] = (cs_t)s;
      }
      for (int j = lane + kWaveSize; j < half; j += kWaveSize) {
        float c, s;
        angle_cos_sin(pp, tab.inv[j], c, s);
        lc[j] = (cs_t)c;
        ls[j] = (cs_t)s;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if constexpr (CS == kCsFromPositions) {
      const int n = ntok * half;
      const int n_pre = kPrePosPath ? kPrePos : 0;
#pragma unroll
      for (int m = 0; m < n_pre; ++m) {
        const int idx = lane + m * kWaveSize;
        if (idx < n) {
          const int tl = idx / half;
          const int j = idx - tl * half;
          const int32_t pp = pos_pre[m];
          float c, s;
          if (p.cs_cache != nullptr && (uint32_t)pp < (uint32_t)p.cache_rows) {
            cached_cos_sin(p.cs_cache, (int64_t)pp * p.n_freq + tab.fidx[j], c, s);
          } else {
            angle_cos_sin(pp, inv_pre[m], c, s);
          }
          lc[idx] = (cs_t)c;
          ls[idx] = (cs_t)s;
        }
      }
      for (int idx = lane + n_pre * kWaveSize; idx < n; idx += kWaveSize) {
        const int tl = idx / half;
        const int j = idx - tl * half;
        const int32_t pp = p.pos[(int64_t)tab.axis[j] * p.pos_stride + t0 + tl];
        float c, s;
        if (p.cs_cache != nullptr && (uint32_t)pp < (uint32_t)p.cache_rows) {
          // the cache holds the same rounded values the computation gives
          cached_cos_sin(p.cs_cache, (int64_t)pp * p.n_freq + tab.fidx[j], c, s);
        } else {
          angle_cos_sin(pp, tab.inv[j], c, s);
        }
        lc[idx] = (cs_t)c;
        ls[idx] = (cs_t)s;
      }
      // LDS traffic of one wavefront is processed in order; this only keeps
      // the compiler from moving the reads above the writes.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    if constexpr (CS == kCsDecode || kPrePosPath) {
      if (s_pre >= 0) {
        if constexpr (CS == kCsDecode) {
          if (s_pre == 1) st_pre.ry = k_cache_buffer(dec_seq, dec_slot);
        }
        float wa[V], wb[V];
        if constexpr (NORM) {
          unpack<BF16, V>(w_pre_a, wa);
          unpack<BF16, V>(w_pre_b, wb);
        }
        finish_steps<BF16, V, CS, NORM, LPR, PREC, 1>(st_pre, L_pre, p, lpr, rot, ca, cb, col_a,
                                                      wa, wb, lc, ls, t0);
        if constexpr (kPrePosPath) {
#pragma unroll
          for (int u = 0; u < kPreSteps - 1; ++u)
            finish_steps<BF16, V, CS, NORM, LPR, PREC, 1>(st_pre, L_more[u], p, lpr, rot, ca, cb,
                                                          col_a, wa, wb, lc, ls, t0);
        }
      }
    }
#pragma unroll 1
    for (int s = 0; s < kSlots; ++s) {
      const int H = p.heads[s];
      if (H == 0) continue;
      // This part's steps of tensor s.
      int lo = (step_begin > pre[s] ? step_begin : pre[s]) - pre[s];
      const int hi = (step_end < pre[s + 1] ? step_end : pre[s + 1]) - pre[s];
      if (s == s_pre) lo += n_pre_steps;   // loaded and finished around the prologue
      if (lo >= hi) continue;
      SlotState<CB> st = make_state(s, lo);
      if constexpr (CS == kCsDecode) {
        if (s == 1) st.ry = k_cache_buffer(dec_seq, dec_slot);
      }

      // The third tensor (v of a packed qkv) is copied: no norm, no rotation.
      if constexpr (CS == kCsFromPositions) {
        if (s == 2) {
          const float none[V] = {};
          const int full = (hi - lo) / U;
          int r0 = lo * rpw;
          for (int g = 0; g < full; ++g, r0 += U * rpw)
            process_steps<BF16, V, kCsNone, false, LPR, PREC, U>(st, r0, p, grp, rpw, lpr,
                                                                 lane_on, false, ca, cb, col_a,
                                                                 none, none, lc, ls, t0);
          for (; r0 < hi * rpw; r0 += rpw)
            process_steps<BF16, V, kCsNone, false, LPR, PREC, 1>(st, r0, p, grp, rpw, lpr,
                                                                 lane_on, false, ca, cb, col_a,
                                                                 none, none, lc, ls, t0);
          continue;
        }
      }

      float wa[V], wb[V];
      int first = 0;
      if constexpr (NORM) {
        if (s != s_pre) {
          // The weights and the first row-step go out together: one round
          // trip instead of two (0.3-0.4% on the RMSNorm workloads).  The
          // preloaded tensor keeps full batches, which measured faster there.
          Words<CB> wra, wrb;
          const __amdgpu_buffer_rsrc_t rw = buffer_of(p.w[s], (uint32_t)(p.D * ES));
          buf_load<CB>(rw, ca, wra);
          buf_load<CB>(rw, cb, wrb);
          StepLoads<CB, 1> L0;
          load_steps<CB, 1>(st, lo * rpw, grp, rpw, lane_on, ca, cb, L0);
          unpack<BF16, V>(wra, wa);
          unpack<BF16, V>(wrb, wb);
          finish_steps<BF16, V, CS, NORM, LPR, PREC, 1>(st, L0, p, lpr, rot, ca, cb, col_a, wa,
                                                        wb, lc, ls, t0);
          first = 1;
        } else {
          Words<CB> r;
          load_words<CB>(static_cast<const char*>(p.w[s]) + (int64_t)col_a * ES, r);
          unpack<BF16, V>(r, wa);
          load_words<CB>(static_cast<const char*>(p.w[s]) + (int64_t)col_b * ES, r);
          unpack<BF16, V>(r, wb);
        }
      }

      // Full batches of U row-steps, then single steps for the remainder.
      const int full = (hi - lo - first) / U;
      int r0 = (lo + first) * rpw;
      for (int g = 0; g < full; ++g, r0 += U * rpw)
        process_steps<BF16, V, CS, NORM, LPR, PREC, U>(st, r0, p, grp, rpw, lpr, lane_on, rot, ca, cb,
                                                 col_a, wa, wb, lc, ls, t0);
      for (; r0 < hi * rpw; r0 += rpw)
        process_steps<BF16, V, CS, NORM, LPR, PREC, 1>(st, r0, p, grp, rpw, lpr, lane_on, rot, ca, cb,
                                                 col_a, wa, wb, lc, ls, t0);
    }
  }
}

// ---------------------------------------------------------------------------
// The staged q/k kernel (no RMSNorm, cos/sin from positions).  A block owns G
// consecutive tokens.  It copies their q and k rows into LDS with direct
// buffer-to-LDS loads (one wavefront instruction moves 64 chunks of 16 bytes,
// consecutive in LDS) and forms the G tokens' cos/sin; the copied tensor (v)
// skips LDS, each lane loading its 16-byte chunks in output order straight
// into registers.  After one barrier it writes v, then q and k rotated, 16
// bytes per lane in output order: in head-major order the G rows of a head go
// out back to back, one contiguous run per plane, and in token-major order a
// token's heads do.  This is the layout transposition of the vision tower's
// packed qkv into per-head planes.  Keeping v out of LDS lets eight blocks
// share a compute unit instead of five.
// Requirements (checked by the host): 16-byte aligned bases, strides and row
// widths (D * ES), an even rotary half, at most kStageV * 256 chunks of v per
// block.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;

// floor(n / d) for n < 2^23 through the binary32 reciprocal inv ~ 1/d,
// corrected to the exact quotient.
__device__ __forceinline__ int div_small(int n, int d, float inv) {
  int q = (int)((float)n * inv);
  if (q * d > n) --q;
  if ((q + 1) * d <= n) ++q;
  return q;
}

// Bytes of LDS a slot's G token-rows take, padded to whole 1 KB wavefront
// transfers so that no lane of the last transfer writes past the region.
__host__ __device__ __forceinline__ int stage_slot_bytes(int G, int heads, int D, int es) {
  const int chunks = G * heads * D * es / 16;
  return ((chunks + kWaveSize - 1) / kWaveSize) * kWaveSize * 16;
}

// The copied tensor (v) skips LDS: each lane loads its 16-byte chunks in
// output order straight into registers, kStageV of them at most.
constexpr int kStageV = 3;
constexpr int kStageLdsSlots = 2;     // q and k go through LDS

// Output chunk k (k >= 0) of a tensor with H heads in a group: head h, token
// g, chunk c; head-major order runs over (h, g, c), token-major over (g, h, c).
struct StageChunk {
  int h, g, c;
};

template <int G>
__device__ __forceinline__ StageChunk stage_split(int k, int cpr, float inv_cpr, int H,
                                                  float inv_h, bool head_major) {
  const int o = div_small(k, cpr, inv_cpr);
  const int hh = (int)((uint32_t)o / (uint32_t)G);
  const int gt = div_small(o, H, inv_h);
  StageChunk r;
  r.c = k - o * cpr;
  r.h = head_major ? hh : o - gt * H;
  r.g = head_major ? o - hh * G : gt;
  return r;
}

template <bool BF16, int PREC, int G>
__global__ void __launch_bounds__(kBlockThreads) stage_kernel(const QKParams p, const ColTable tab) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EC = 16 / ES;          // elements per 16-byte chunk
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWaveSize - 1);
  const int wib = __builtin_amdgcn_readfirstlane(tid / kWaveSize);
  const int64_t t0 = (int64_t)blockIdx.x * G;
  const int64_t left = p.T - t0;
  const int nvalid = left < G ? (int)left : G;
  const int D = p.D, half = p.half, rd = p.rd;
  const int cpr = D * ES / 16;         // chunks per head row

  int lds_off[kStageLdsSlots];
  int off = 0;
#pragma unroll
  for (int s = 0; s < kStageLdsSlots; ++s) {
    lds_off[s] = off;
    if (p.heads[s] > 0) off += stage_slot_bytes(G, p.heads[s], D, ES);
  }
  float2* cs = reinterpret_cast<float2*>(smem + off);   // [G][half]
  const float inv_cpr = p.inv_cpr;

  // 1. token rows of q and k to LDS, in memory order [g][head][D]
#pragma unroll 1
  for (int s = 0; s < kStageLdsSlots; ++s) {
    const int H = p.heads[s];
    if (H == 0) continue;
    const int rcs = H * cpr;                            // chunks per token
    const int nch = G * rcs;
    const uint32_t tsb = (uint32_t)(p.x_ts[s] * ES);    // token stride, bytes
    const __amdgpu_buffer_rsrc_t rx = buffer_of(
        static_cast<const char*>(p.x[s]) + t0 * p.x_ts[s] * ES,
        (uint32_t)(nvalid - 1) * tsb + (uint32_t)rcs * 16u);
    const float inv = 1.0f / (float)rcs;
    unsigned char* dst = smem + lds_off[s];
#pragma unroll 1
    for (int kb = wib * kWaveSize; kb < nch; kb += kBlockThreads) {
      const int k = kb + lane;
      const int g = div_small(k, rcs, inv);
      const uint32_t vo = k < nch && g < nvalid ? (uint32_t)g * tsb + (uint32_t)(k - g * rcs) * 16u
                                                : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(dst + kb * 16), 16, vo, 0, 0, 0);
    }
  }

  // 2. cos/sin of the block's tokens (tokens past T repeat the last one)
  {
    const float inv = 1.0f / (float)half;
#pragma unroll 1
    for (int i = tid; i < G * half; i += kBlockThreads) {
      const int g = div_small(i, half, inv);
      const int j = i - g * half;
      const int64_t t = t0 + (g < nvalid ? g : nvalid - 1);
      const int32_t pp = p.pos[(int64_t)tab.axis[j] * p.pos_stride + t];
      float c, sn;
      if (p.cs_cache != nullptr && (uint32_t)pp < (uint32_t)p.cache_rows) {
        const float2 v = *reinterpret_cast<const float2*>(
            p.cs_cache + 2 * ((int64_t)pp * p.n_freq + tab.fidx[j]));
        c = v.x;
        sn = v.y;
      } else {
        angle_cos_sin(pp, tab.inv[j], c, sn);
      }
      cs[i] = make_float2(c, sn);
    }
  }
  // 2b. v chunks in output order to registers
  Words<16> rv[kStageV];
  {
    const int H = p.heads[2];
    const int nch = H * G * cpr;
    const uint32_t tsb = (uint32_t)(p.x_ts[2] * ES);
    const __amdgpu_buffer_rsrc_t rx = buffer_of(
        static_cast<const char*>(p.x[2]) + t0 * p.x_ts[2] * ES,
        H > 0 ? (uint32_t)(nvalid - 1) * tsb + (uint32_t)(H * cpr) * 16u : 0u);
#pragma unroll
    for (int j = 0; j < kStageV; ++j) {
      const int k = tid + j * kBlockThreads;
      const StageChunk q = stage_split<G>(k < nch ? k : 0, cpr, inv_cpr, H > 0 ? H : 1,
                                          p.inv_heads[2], p.stage_hm != 0);
      const bool ok = k < nch && q.g < nvalid;
      buf_load<16>(rx, ok ? (uint32_t)q.g * tsb + (uint32_t)(q.h * cpr + q.c) * 16u : kOutOfRange,
                   rv[j]);
    }
  }

  // every load has landed (the LDS transfers among them), and the LDS
  // writes of the cos/sin; waiting for the v chunks too costs nothing measurable
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // 3. v from registers
  {
    const int H = p.heads[2];
    const int nch = H * G * cpr;
    const __amdgpu_buffer_rsrc_t ry = buffer_of(
        static_cast<char*>(p.y[2]) + t0 * p.y_ts[2] * ES,
        H > 0 ? (uint32_t)(((int64_t)(H - 1) * p.y_hs[2] + (int64_t)(nvalid - 1) * p.y_ts[2] + D)
                           * ES) : 0u);
#pragma unroll
    for (int j = 0; j < kStageV; ++j) {
      const int k = tid + j * kBlockThreads;
      const StageChunk q = stage_split<G>(k < nch ? k : 0, cpr, inv_cpr, H > 0 ? H : 1,
                                          p.inv_heads[2], p.stage_hm != 0);
      const uint32_t yo = k < nch && q.g < nvalid
          ? (uint32_t)(((int64_t)q.h * p.y_hs[2] + (int64_t)q.g * p.y_ts[2]) * ES) +
                (uint32_t)q.c * 16u
          : kOutOfRange;
      buf_store<BF16, 16>(ry, yo, rv[j]);
    }
  }

  // 4. rotate q and k.  Thread t owns one 16-byte chunk position (token g,
  // chunk c) of the group's rows, pos = t % (G * cpr), and walks the heads
  // h = t / (G * cpr), + hl, + 2 hl, ... (hl = 256 / (G * cpr) threads per
  // position; the host keeps G * cpr <= 256).  Its columns, partner offsets
  // and cos/sin are fixed, so they are formed once; per chunk there remain
  // the LDS reads, the rotation and the store, and for each head the
  // positions of a group go out as one contiguous run.
  {
    const int gc = G * cpr;
    const int hl = kBlockThreads / gc;
    const int h0 = tid / gc;
    const int pos = tid - h0 * gc;
    const int g = pos / cpr;
    const int c = pos - g * cpr;
    constexpr int NP = EC / 2;           // element pairs per chunk
    constexpr int WP = BF16 ? 1 : 2;     // 32-bit words per pair
    bool rot[NP];
    int poff[NP];                        // byte offset of the partner pair in the row
    double cd[EC], sd[EC];               // cos, and sin with the half's sign
    float cf[EC], sf[EC];
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int col = c * EC + 2 * m;
      rot[m] = col < rd;
      const bool first = col < half;
      const int pcol = !rot[m] ? col : (first ? col + half : col - half);
      const int j = !rot[m] ? 0 : (first ? col : col - half);
      poff[m] = pcol * ES;
      const float4 cc = *reinterpret_cast<const float4*>(cs + g * half + j);
      const float cv[2] = {cc.x, cc.z};
      const float sv[2] = {cc.y, cc.w};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float cfe = cv[e], sfe = sv[e];
        if constexpr (BF16 && PREC == MROPE_PRECISION_DTYPE) {
          cfe = round_bf16(cfe);
          sfe = round_bf16(sfe);
        }
        // first half: y c - partner s = y c + partner (-s); negating is exact
        cf[2 * m + e] = cfe;
        sf[2 * m + e] = first ? -sfe : sfe;
        cd[2 * m + e] = (double)cv[e];
        sd[2 * m + e] = first ? -(double)sv[e] : (double)sv[e];
      }
    }
#pragma unroll 1
    for (int s = 0; s < kStageLdsSlots; ++s) {
      const int H = p.heads[s];
      if (H == 0 || h0 >= hl) continue;
      const __amdgpu_buffer_rsrc_t ry = buffer_of(
          static_cast<char*>(p.y[s]) + t0 * p.y_ts[s] * ES,
          (uint32_t)(((int64_t)(H - 1) * p.y_hs[s] + (int64_t)(nvalid - 1) * p.y_ts[s] + D) * ES));
      const unsigned char* row = smem + lds_off[s] + (g * H + h0) * (D * ES);
      const int row_step = hl * D * ES;
      uint32_t yo = (uint32_t)(((int64_t)h0 * p.y_hs[s] + (int64_t)g * p.y_ts[s]) * ES) +
                    (uint32_t)c * 16u;
      const uint32_t y_step = (uint32_t)((int64_t)hl * p.y_hs[s] * ES);
      const bool live = g < nvalid;
#pragma unroll 1
      for (int h = h0; h < H; h += hl, row += row_step, yo += y_step) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + c * 16);
        Words<16> own;
        own.w[0] = v.x; own.w[1] = v.y; own.w[2] = v.z; own.w[3] = v.w;
        float a[EC], b[EC];
        unpack<BF16, EC>(own, a);
#pragma unroll
        for (int m = 0; m < NP; ++m) {
          if constexpr (BF16) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(row + poff[m]);
            b[2 * m] = bf_lo(w);
            b[2 * m + 1] = bf_hi(w);
          } else {
            const float2 w = *reinterpret_cast<const float2*>(row + poff[m]);
            b[2 * m] = w.x;
            b[2 * m + 1] = w.y;
          }
        }
#pragma unroll
        for (int i = 0; i < EC; ++i) {
          if constexpr (PREC == MROPE_PRECISION_EXACT) {
            a[i] = (float)__builtin_fma((double)a[i], cd[i], (double)b[i] * sd[i]);
          } else {
#pragma clang fp contract(off)
            float po = a[i] * cf[i];
            float pq = b[i] * sf[i];
            if constexpr (BF16 && PREC == MROPE_PRECISION_DTYPE) {
              po = round_bf16(po);
              pq = round_bf16(pq);
            }
            a[i] = po + pq;
          }
        }
        Words<16> out;
        pack<BF16, EC>(a, out);
#pragma unroll
        for (int m = 0; m < NP; ++m)
#pragma unroll
          for (int w = 0; w < WP; ++w)
            out.w[m * WP + w] = rot[m] ? out.w[m * WP + w] : own.w[m * WP + w];
        buf_store<BF16, 16>(ry, live ? yo : kOutOfRange, out);
      }
    }
  }
}

template <bool BF16, int PREC, int G>
int launch_stage_t(const QKParams& p, const ColTable& tab, hipStream_t st) {
  constexpr int ES = BF16 ? 2 : 4;
  const int64_t blocks = (p.T + G - 1) / G;
  int lds = G * p.half * (int)sizeof(float2);
  for (int s = 0; s < kStageLdsSlots; ++s)
    if (p.heads[s] > 0) lds += stage_slot_bytes(G, p.heads[s], p.D, ES);
  if (lds > kLdsPerCu) return (int)hipErrorInvalidValue;
  if (p.waves_cap > 0) {
    const int cap_lds = (kLdsPerCu / p.waves_cap) & ~511;
    if (cap_lds > lds) lds = cap_lds;
  }
  hipLaunchKernelGGL((stage_kernel<BF16, PREC, G>), dim3((unsigned)blocks), dim3(kBlockThreads),
                     lds, st, p, tab);
  return (int)hipGetLastError();
}

template <bool BF16, int G>
int launch_stage_g(int prec, const QKParams& p, const ColTable& tab, hipStream_t st) {
  switch (prec) {
    case MROPE_PRECISION_EXACT: return launch_stage_t<BF16, MROPE_PRECISION_EXACT, G>(p, tab, st);
    case MROPE_PRECISION_DTYPE: return launch_stage_t<BF16, MROPE_PRECISION_DTYPE, G>(p, tab, st);
    case MROPE_PRECISION_FP32:
      if constexpr (BF16) return launch_stage_t<BF16, MROPE_PRECISION_FP32, G>(p, tab, st);
      break;
  }
  return (int)hipErrorInvalidValue;
}

template <bool BF16>
int launch_stage_d(int prec, int G, const QKParams& p, const ColTable& tab, hipStream_t st) {
  switch (G) {
    case 1: return launch_stage_g<BF16, 1>(prec, p, tab, st);
    case 2: return launch_stage_g<BF16, 2>(prec, p, tab, st);
    case 4: return launch_stage_g<BF16, 4>(prec, p, tab, st);
    case 8: return launch_stage_g<BF16, 8>(prec, p, tab, st);
    case 16: return launch_stage_g<BF16, 16>(prec, p, tab, st);
  }
  return (int)hipErrorInvalidValue;
}

// cos/sin tables [T][rd]: one thread per (token, column < half).
__global__ void __launch_bounds__(256) cos_sin_kernel(const CosSinParams p, const ColTable tab) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.T * p.half) return;
  const int64_t t = idx / p.half;
  const int j = (int)(idx - t * p.half);
  const int32_t pp = p.pos[(int64_t)tab.axis[j] * p.pos_stride + t];
  float c, s;
  angle_cos_sin(pp, tab.inv[j], c, s);
  float* cr = p.cos + t * p.cs_ts;
  float* sr = p.sin + t * p.cs_ts;
  cr[j] = c;
  cr[j + p.half] = c;
  sr[j] = s;
  sr[j + p.half] = s;
}

// cos/sin cache by position: one thread per (position, frequency).
__global__ void __launch_bounds__(256) cos_sin_cache_kernel(const ColTable tab, int n_freq,
                                                            int64_t n, float* cache) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int64_t pos = idx / n_freq;
  const int i = (int)(idx - pos * n_freq);
  float c, s;
  angle_cos_sin((int32_t)pos, tab.inv[i], c, s);
  float2 v;
  v.x = c;
  v.y = s;
  *reinterpret_cast<float2*>(cache + 2 * idx) = v;
}

template <bool BF16, int V, int CS, bool NORM, int LPR, int PREC>
int launch_t(QKParams p, const ColTable& tab, int nt_cap, hipStream_t st) {
  const bool cs_lds = CS == kCsFromPositions || CS == kCsDecode;
  if (CS == kCsFromPositions) fit_axis_rule(tab, p.half, p);
  p.nt = nt_cap;   // tokens per wavefront, chosen by the host
  if (p.nt < 1 || CS == kCsDecode) p.nt = 1;
  for (int s = 0; s < kSlots; ++s) {
    const int H = p.heads[s] > 0 ? p.heads[s] : 1;
    p.dq[s] = p.rpw / H;
    p.dr[s] = p.rpw - p.dq[s] * H;
    p.inv_heads[s] = 1.0f / (float)H;
  }
  // Small launches split each tile's row-steps over several wavefronts so
  // that about kMinWaves are in flight; large ones keep one per tile.
  const int64_t tiles = (p.T + p.nt - 1) / p.nt;
  int tile_steps = 0;
  for (int s = 0; s < kSlots; ++s) tile_steps += (p.nt * p.heads[s] + p.rpw - 1) / p.rpw;
  int64_t parts = (kMinWaves + tiles - 1) / tiles;
  if (parts > tile_steps) parts = tile_steps;
  if (parts < 1) parts = 1;
  p.parts = (int)parts;
  const int64_t waves = tiles * parts;
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  int lds = cs_lds ? kWavesPerBlock * 2 * p.nt * p.half * (int)sizeof(float) : 0;
  if (p.waves_cap > 0) {
    // Bound the resident wavefronts per SIMD: a block asks for enough LDS
    // that at most waves_cap blocks of four wavefronts share a compute unit.
    const int cap_lds = (kLdsPerCu / p.waves_cap) & ~511;
    if (cap_lds > lds) lds = cap_lds;
  }
  hipLaunchKernelGGL((qk_kernel<BF16, V, CS, NORM, LPR, PREC>), dim3((unsigned)blocks),
                     dim3(kBlockThreads), lds, st, p, tab);
  return (int)hipGetLastError();
}

template <bool BF16, int V, int LPR, int PREC>
int launch_rotating(int cs_mode, bool norm, const QKParams& p, const ColTable& tab, int nt_cap,
                    hipStream_t st) {
  if (cs_mode == kCsFromPositions)
    return norm ? launch_t<BF16, V, kCsFromPositions, true, LPR, PREC>(p, tab, nt_cap, st)
                : launch_t<BF16, V, kCsFromPositions, false, LPR, PREC>(p, tab, nt_cap, st);
  if (cs_mode == kCsDecode)
    return norm ? launch_t<BF16, V, kCsDecode, true, LPR, PREC>(p, tab, nt_cap, st)
                : launch_t<BF16, V, kCsDecode, false, LPR, PREC>(p, tab, nt_cap, st);
  if (cs_mode == kCsFromTable && !norm)
    return launch_t<BF16, V, kCsFromTable, false, LPR, PREC>(p, tab, nt_cap, st);
  return (int)hipErrorInvalidValue;
}

template <bool BF16, int V, int LPR>
int launch_mode(int cs_mode, bool norm, int prec, const QKParams& p, const ColTable& tab,
                int nt_cap, hipStream_t st) {
  if (cs_mode == kCsNone)
    return norm ? launch_t<BF16, V, kCsNone, true, LPR, MROPE_PRECISION_EXACT>(p, tab, nt_cap, st)
                : (int)hipErrorInvalidValue;
  switch (prec) {
    case MROPE_PRECISION_EXACT:
      return launch_rotating<BF16, V, LPR, MROPE_PRECISION_EXACT>(cs_mode, norm, p, tab, nt_cap, st);
    case MROPE_PRECISION_DTYPE:
      return launch_rotating<BF16, V, LPR, MROPE_PRECISION_DTYPE>(cs_mode, norm, p, tab, nt_cap, st);
    case MROPE_PRECISION_FP32:
      // binary32 tensors arrive as DTYPE (the same arithmetic)
      if constexpr (BF16)
        return launch_rotating<BF16, V, LPR, MROPE_PRECISION_FP32>(cs_mode, norm, p, tab, nt_cap,
                                                                   st);
      break;
  }
  return (int)hipErrorInvalidValue;
}

// 16-byte chunks with a power-of-two lane count per row get a kernel with the
// lane count fixed at compile time; everything else takes the runtime form.
template <bool BF16, int V>
int launch_lpr(int cs_mode, bool norm, int prec, const QKParams& p, const ColTable& tab,
               int nt_cap, hipStream_t st) {
  if constexpr (V * (BF16 ? 2 : 4) == 16) {
    switch (p.lpr) {
      case 2: return launch_mode<BF16, V, 2>(cs_mode, norm, prec, p, tab, nt_cap, st);
      case 4: return launch_mode<BF16, V, 4>(cs_mode, norm, prec, p, tab, nt_cap, st);
      case 8: return launch_mode<BF16, V, 8>(cs_mode, norm, prec, p, tab, nt_cap, st);
      case 16: return launch_mode<BF16, V, 16>(cs_mode, norm, prec, p, tab, nt_cap, st);
      case 32: return launch_mode<BF16, V, 32>(cs_mode, norm, prec, p, tab, nt_cap, st);
      default: break;
    }
  }
  return launch_mode<BF16, V, 0>(cs_mode, norm, prec, p, tab, nt_cap, st);
}

}  // namespace

int launch_qk(int dtype, int vec, int cs_mode, bool norm, int prec, const QKParams& p,
              const ColTable& tab, int nt_cap, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == MROPE_DTYPE_BF16) {
    switch (vec) {
      case 8: return launch_lpr<true, 8>(cs_mode, norm, prec, p, tab, nt_cap, st);
      case 4: return launch_lpr<true, 4>(cs_mode, norm, prec, p, tab, nt_cap, st);
      case 2: return launch_lpr<true, 2>(cs_mode, norm, prec, p, tab, nt_cap, st);
      case 1: return launch_lpr<true, 1>(cs_mode, norm, prec, p, tab, nt_cap, st);
    }
  } else {
    switch (vec) {
      case 4: return launch_lpr<false, 4>(cs_mode, norm, prec, p, tab, nt_cap, st);
      case 2: return launch_lpr<false, 2>(cs_mode, norm, prec, p, tab, nt_cap, st);
      case 1: return launch_lpr<false, 1>(cs_mode, norm, prec, p, tab, nt_cap, st);
    }
  }
  return (int)hipErrorInvalidValue;
}

int launch_stage(int dtype, int prec, int G, const QKParams& p, const ColTable& tab,
                 void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  return dtype == MROPE_DTYPE_BF16 ? launch_stage_d<true>(prec, G, p, tab, st)
                                   : launch_stage_d<false>(prec, G, p, tab, st);
}

int stage_lds_bytes(int dtype, int G, const QKParams& p) {
  const int es = dtype == MROPE_DTYPE_BF16 ? 2 : 4;
  int lds = G * p.half * 8;
  for (int s = 0; s < kStageLdsSlots; ++s)
    if (p.heads[s] > 0) lds += stage_slot_bytes(G, p.heads[s], p.D, es);
  return lds;
}

int stage_max_v_chunks() { return kStageV * kBlockThreads; }

int launch_cos_sin_cache(const ColTable& tab, int n_freq, int rows, float* cache, void* stream) {
  const int64_t n = (int64_t)rows * n_freq;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(cos_sin_cache_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), tab, n_freq, n, cache);
  return (int)hipGetLastError();
}

int launch_cos_sin(const CosSinParams& p, const ColTable& tab, void* stream) {
  const int64_t n = p.T * p.half;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(cos_sin_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p, tab);
  return (int)hipGetLastError();
}

}  // namespace mrope
