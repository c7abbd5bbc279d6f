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
//    instruction and U rows in flight per lane.
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

#include "mrope_internal.h"

namespace mrope {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Chunk storage: V elements of 2 (bf16) or 4 (fp32) bytes, as 32-bit words.
// ---------------------------------------------------------------------------

template <int CB>
struct Words {
  static constexpr int N = CB >= 4 ? CB / 4 : 1;
  uint32_t w[N];
};

template <int CB>
__device__ __forceinline__ void load_words(const char* p, Words<CB>& r) {
  if constexpr (CB == 16) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (CB == 8) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else if constexpr (CB == 4) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else {
    r.w[0] = *reinterpret_cast<const uint16_t*>(p);
  }
}

template <int CB>
__device__ __forceinline__ void store_words(char* p, const Words<CB>& r) {
  if constexpr (CB == 16) {
    u32x4_t v = {r.w[0], r.w[1], r.w[2], r.w[3]};
    *reinterpret_cast<u32x4_t*>(p) = v;
  } else if constexpr (CB == 8) {
    u32x2_t v = {r.w[0], r.w[1]};
    *reinterpret_cast<u32x2_t*>(p) = v;
  } else if constexpr (CB == 4) {
    *reinterpret_cast<uint32_t*>(p) = r.w[0];
  } else {
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)r.w[0];
  }
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Round two binary32 values to bfloat16 (nearest even, v_cvt_pk_bf16_f32) and
// return them packed, first value in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Round two binary32 values to bfloat16 in place (kept as binary32).
__device__ __forceinline__ void round_bf16_pair(float& a, float& b) {
  const uint32_t u = pack_bf16(a, b);
  a = bf_lo(u);
  b = bf_hi(u);
}

template <bool BF16, int V>
__device__ __forceinline__ void unpack(const Words<(BF16 ? 2 : 4) * V>& r, float (&x)[V]) {
  if constexpr (BF16) {
    if constexpr (V == 1) {
      x[0] = bf_lo(r.w[0]);
    } else {
#pragma unroll
      for (int i = 0; i < V / 2; ++i) {
        x[2 * i] = bf_lo(r.w[i]);
        x[2 * i + 1] = bf_hi(r.w[i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) x[i] = __builtin_bit_cast(float, r.w[i]);
  }
}

template <bool BF16, int V>
__device__ __forceinline__ void pack(const float (&x)[V], Words<(BF16 ? 2 : 4) * V>& r) {
  if constexpr (BF16) {
    if constexpr (V == 1) {
      r.w[0] = pack_bf16(x[0], 0.0f) & 0xFFFFu;
    } else {
#pragma unroll
      for (int i = 0; i < V / 2; ++i) r.w[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) r.w[i] = __builtin_bit_cast(uint32_t, x[i]);
  }
}

// Round the 2V values of a lane (two chunks) to bfloat16, kept as binary32.
template <int V>
__device__ __forceinline__ void round_bf16_chunks(float (&a)[V], float (&b)[V]) {
  if constexpr (V == 1) {
    round_bf16_pair(a[0], b[0]);
  } else {
#pragma unroll
    for (int i = 0; i < V; i += 2) {
      round_bf16_pair(a[i], a[i + 1]);
      round_bf16_pair(b[i], b[i + 1]);
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-lane sum of a float64 over the lpr lanes of a row.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  int lo = (int)(uint32_t)u;
  int hi = (int)(uint32_t)(u >> 32);
  lo = __builtin_amdgcn_update_dpp(0, lo, CTRL, 0xF, 0xF, false);
  hi = __builtin_amdgcn_update_dpp(0, hi, CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// All lanes of the wavefront must be active.  Each step adds the partner's
// value, which is commutative, so every lane of a group ends with the same sum.
__device__ __forceinline__ double group_sum(double v, int lpr) {
  if ((lpr & (lpr - 1)) == 0) {
    if (lpr >= 2) v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    if (lpr >= 4) v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    if (lpr >= 8) v += dpp_f64<0x141>(v);  // row_half_mirror: other quad of 8
    if (lpr >= 16) v += dpp_f64<0x140>(v); // row_mirror: other half of 16
    if (lpr >= 32) v += __shfl_xor(v, 16);
    if (lpr >= 64) v += __shfl_xor(v, 32);
    return v;
  }
  // Rows whose lane count is not a power of two: every lane adds the group's
  // partials in lane order.
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int base = (lane / lpr) * lpr;
  double s = 0.0;
  for (int i = 0; i < lpr; ++i) s += __shfl(v, (base + i) & (kWaveSize - 1));
  return s;
}

// fl32 of 1/sqrt(m): hardware estimate refined by two Newton steps in double;
// the result is within a few double ulps of the exact value before rounding.
__device__ __forceinline__ float rsqrt_to_f32(double m) {
  double y = __builtin_amdgcn_rsq(m);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double t = m * y;
    const double e = __builtin_fma(-t, y, 1.0);      // 1 - m y^2
    y = __builtin_fma(0.5 * y, e, y);
  }
  return (float)y;
}

// cos/sin of the binary32 angle float(p) * inv, in double, rounded once.
__device__ __forceinline__ void angle_cos_sin(int32_t pos, float inv, float& c, float& s) {
  const float a = __fmul_rn((float)pos, inv);
  double sd, cd;
  sincos((double)a, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// ---------------------------------------------------------------------------
// The q/k kernel.
// ---------------------------------------------------------------------------

template <bool BF16, int V, int CS, bool NORM>
__global__ void __launch_bounds__(kBlockThreads)
qk_kernel(const QKParams p, const ColTable tab) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int CB = ES * V;
  constexpr int U = 4;  // rows in flight per lane
  extern __shared__ float lds[];

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wib = threadIdx.x / kWaveSize;
  const int half = p.half;
  float* lc = lds + wib * (2 * p.nt * half);
  float* ls = lc + p.nt * half;

  const int lpr = p.lpr;
  const int grp = lane / lpr;
  const int l = lane - grp * lpr;
  const bool lane_on = grp < p.rpw;
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

  const int64_t wstride = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t tile = (int64_t)blockIdx.x * kWavesPerBlock + wib; tile < p.ntiles;
       tile += wstride) {
    const int64_t t0 = tile * p.nt;
    const int ntok = (int)((p.T - t0) < p.nt ? (p.T - t0) : p.nt);

    if constexpr (CS == kCsFromPositions) {
      const int n = ntok * half;
      for (int idx = lane; idx < n; idx += kWaveSize) {
        const int tl = idx / half;
        const int j = idx - tl * half;
        const int32_t pp = p.pos[(int64_t)tab.axis[j] * p.pos_stride + t0 + tl];
        angle_cos_sin(pp, tab.inv[j], lc[idx], ls[idx]);
      }
      // LDS traffic of one wavefront is processed in order; this only keeps
      // the compiler from moving the reads above the writes.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

#pragma unroll 1
    for (int s = 0; s < 2; ++s) {
      const int H = p.heads[s];
      if (H == 0) continue;
      const int nrows = ntok * H;
      const char* xb = static_cast<const char*>(p.x[s]);
      char* yb = static_cast<char*>(p.y[s]);
      const int64_t xts = p.x_ts[s];
      const int64_t yts = p.y_ts[s];

      float wa[V], wb[V];
      if constexpr (NORM) {
        Words<CB> r;
        load_words<CB>(static_cast<const char*>(p.w[s]) + (int64_t)col_a * ES, r);
        unpack<BF16, V>(r, wa);
        load_words<CB>(static_cast<const char*>(p.w[s]) + (int64_t)col_b * ES, r);
        unpack<BF16, V>(r, wb);
      }

      // (token, head) of this lane's row, advanced by rpw rows per step.
      int tl = grp / H;
      int h = grp - tl * H;
      const int dq = p.rpw / H;
      const int dr = p.rpw - dq * H;

      for (int r0 = 0; r0 < nrows; r0 += U * p.rpw) {
        Words<CB> ra[U], rb[U];
        int tlu[U];
        bool ok[U];
        int64_t yoff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = r0 + u * p.rpw + grp;
          ok[u] = lane_on && r < nrows;
          tlu[u] = tl;
          const int64_t xoff = (t0 + tl) * xts + (int64_t)h * p.D;
          yoff[u] = (t0 + tl) * yts + (int64_t)h * p.D;
          if (ok[u]) {
            load_words<CB>(xb + (xoff + col_a) * ES, ra[u]);
            load_words<CB>(xb + (xoff + col_b) * ES, rb[u]);
          } else {
#pragma unroll
            for (int i = 0; i < Words<CB>::N; ++i) ra[u].w[i] = rb[u].w[i] = 0u;
          }
          h += dr;
          tl += dq;
          if (h >= H) {
            h -= H;
            ++tl;
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
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
            ss = group_sum(ss, lpr);
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
              // Rows past the tile's end are computed but not stored; read
              // their cos/sin from the tile's first token so every read stays
              // inside this wavefront's LDS slice and the caller's tables.
              const int tlr = ok[u] ? tlu[u] : 0;
              float ca[V], sa[V], cb[V], sb[V];
              if constexpr (CS == kCsFromPositions) {
                const int o = tlr * half + col_a;
#pragma unroll
                for (int i = 0; i < V; ++i) {
                  ca[i] = lc[o + i];
                  sa[i] = ls[o + i];
                  cb[i] = ca[i];
                  sb[i] = sa[i];
                }
              } else {
                const int64_t o = (t0 + tlr) * p.cs_ts;
#pragma unroll
                for (int i = 0; i < V; ++i) {
                  ca[i] = p.cos[o + col_a + i];
                  sa[i] = p.sin[o + col_a + i];
                  cb[i] = p.cos[o + col_b + i];
                  sb[i] = p.sin[o + col_b + i];
                }
              }
#pragma unroll
              for (int i = 0; i < V; ++i) {
                const double ya = a[i];
                const double yb = b[i];
                const double oa = __builtin_fma(ya, (double)ca[i], -(yb * (double)sa[i]));
                const double ob = __builtin_fma(yb, (double)cb[i], ya * (double)sb[i]);
                a[i] = (float)oa;
                b[i] = (float)ob;
              }
            }
          }

          if (ok[u]) {
            Words<CB> wa_out, wb_out;
            pack<BF16, V>(a, wa_out);
            pack<BF16, V>(b, wb_out);
            store_words<CB>(yb + (yoff[u] + col_a) * ES, wa_out);
            store_words<CB>(yb + (yoff[u] + col_b) * ES, wb_out);
          }
        }
      }
    }
    // The next tile rewrites this wavefront's LDS slice; keep the order.
    __builtin_amdgcn_wave_barrier();
  }
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

template <bool BF16, int V, int CS, bool NORM>
int launch_t(const QKParams& p, const ColTable& tab, int grid, int lds, hipStream_t st) {
  hipLaunchKernelGGL((qk_kernel<BF16, V, CS, NORM>), dim3(grid), dim3(kBlockThreads), lds, st,
                     p, tab);
  return (int)hipGetLastError();
}

template <bool BF16, int V>
int launch_mode(int cs_mode, bool norm, const QKParams& p, const ColTable& tab, int grid,
                int lds, hipStream_t st) {
  if (cs_mode == kCsFromPositions)
    return norm ? launch_t<BF16, V, kCsFromPositions, true>(p, tab, grid, lds, st)
                : launch_t<BF16, V, kCsFromPositions, false>(p, tab, grid, lds, st);
  if (cs_mode == kCsFromTable && !norm)
    return launch_t<BF16, V, kCsFromTable, false>(p, tab, grid, lds, st);
  if (cs_mode == kCsNone && norm)
    return launch_t<BF16, V, kCsNone, true>(p, tab, grid, lds, st);
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_qk(int dtype, int vec, int cs_mode, bool norm, const QKParams& p,
              const ColTable& tab, int grid, int lds_bytes, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == MROPE_DTYPE_BF16) {
    switch (vec) {
      case 8: return launch_mode<true, 8>(cs_mode, norm, p, tab, grid, lds_bytes, st);
      case 4: return launch_mode<true, 4>(cs_mode, norm, p, tab, grid, lds_bytes, st);
      case 2: return launch_mode<true, 2>(cs_mode, norm, p, tab, grid, lds_bytes, st);
      case 1: return launch_mode<true, 1>(cs_mode, norm, p, tab, grid, lds_bytes, st);
    }
  } else {
    switch (vec) {
      case 4: return launch_mode<false, 4>(cs_mode, norm, p, tab, grid, lds_bytes, st);
      case 2: return launch_mode<false, 2>(cs_mode, norm, p, tab, grid, lds_bytes, st);
      case 1: return launch_mode<false, 1>(cs_mode, norm, p, tab, grid, lds_bytes, st);
    }
  }
  return (int)hipErrorInvalidValue;
}

int launch_cos_sin(const CosSinParams& p, const ColTable& tab, void* stream) {
  const int64_t n = p.T * p.half;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(cos_sin_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p, tab);
  return (int)hipGetLastError();
}

}  // namespace mrope
