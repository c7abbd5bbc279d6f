// The group kernel for gfx950 (planes_kernel): the positions path without
// RMSNorm on a packed q/k(/v) input written to per-head planes, with full
// rotary.  A block owns G consecutive tokens and every plane of the launch;
// its threads walk the group's 16-byte chunks in output order, so each
// plane's run of G rows (a whole number of 128-byte lines) is written by
// the block's adjacent lanes.  The arithmetic per element is qk_kernel's
// (mrope_kernels.hip), so the results are bit-identical.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mrope_device.h"

// Non-temporal stores (1) or cached ones (0).  A plane's run is whole lines.
#ifndef MROPE_PLANES_NT_STORES
#define MROPE_PLANES_NT_STORES 1
#endif

namespace mrope {
namespace {

// ---------------------------------------------------------------------------
// One block: G tokens x the P planes of q, k (rotated) and v (copied), each
// plane's run of G rows of D elements = G * cpr chunks of 16 bytes.  The
// chunks of one tensor are spread over the block's threads, chunk f on
// thread f mod kPlanesThreads, in output order (plane, token, chunk).  A
// thread issues every load of its chunks (its own chunk and, for q and k,
// the split-half partner's elements) before the group's cos/sin are formed
// (one sincos per (token, column), through LDS), then rotates and stores.
// Partners: element e < half pairs with e + half, e >= half with e - half;
// a chunk holds V consecutive elements, so its partners are V consecutive
// elements too, except for the chunk that straddles the half (half not a
// multiple of V): its first part pairs with the row's last elements and its
// second part with the row's first ones.  The partner is read as two 8-byte
// pieces at per-lane offsets, which covers both cases (SPLIT), or as one
// 16-byte chunk when half is a multiple of V.
// ---------------------------------------------------------------------------

constexpr int kPlanesThreads = 512;
#ifndef MROPE_PLANES_TASKS
#define MROPE_PLANES_TASKS 3
#endif
constexpr int kPlanesTasks = MROPE_PLANES_TASKS;   // chunks per thread per tensor, at most

template <bool BF16, int PREC, bool SPLIT>
__global__ void __launch_bounds__(kPlanesThreads) planes_kernel(const QKParams p,
                                                               const ColTable tab) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int V = 16 / ES;
  extern __shared__ float2 cs[];      // [G][half] (cos, sin)
  const int tid = threadIdx.x;
  const int G = p.nt;
  const int half = p.half;
  const int D = p.D;
  const int cpr = D / V;
  const int run = G * cpr;            // chunks of one plane's run
  const int64_t t0 = (int64_t)blockIdx.x * G;
  const int nvalid = (int)(p.T - t0 < G ? p.T - t0 : G);

  // 1. What this thread's sincos needs, loaded before the rows (the axis
  // from the rule fitted to the table on the host, so no table load waits
  // ahead of them).
  const int ncs = G * half;
  int cg = 0, cj = 0;
  int32_t pp = 0;
  float inv = 0.0f;
  if (tid < ncs) {
    cg = tid / half;
    cj = tid - cg * half;
    int ax;
    if (p.ax_mode == 0) ax = (cj >= p.ax_a) + (cj >= p.ax_b);
    else if (p.ax_mode == 1) ax = (cj % 3 == 1 && cj < p.ax_a) ? 1 : (cj % 3 == 2 && cj < p.ax_b) ? 2 : 0;
    else ax = tab.axis[cj];
    const int64_t t = t0 + (cg < nvalid ? cg : nvalid - 1);
    pp = p.pos[(int64_t)ax * p.pos_stride + t];
    inv = tab.inv[cj];
  }

  // 2. Every load of the thread's chunks, tensor after tensor.
  Words<16> own[kSlots][kPlanesTasks], par[kSlots][kPlanesTasks];
  uint32_t yoff[kSlots][kPlanesTasks];
  int col[kSlots][kPlanesTasks], tok[kSlots][kPlanesTasks];
  const int hc = half / V;            // chunks wholly in the first half
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int H = p.heads[s];
    const int nch = H * run;
    const __amdgpu_buffer_rsrc_t rx = buffer_of(
        static_cast<const char*>(p.x[s]) + t0 * p.x_ts[s] * ES,
        H > 0 ? (uint32_t)(((int64_t)(G - 1) * p.x_ts[s] + (int64_t)H * D) * ES) : 0u);
#pragma unroll
    for (int u = 0; u < kPlanesTasks; ++u) {
      const int f = tid + u * kPlanesThreads;
      // plane h = f / run, token g, chunk c: binary32 reciprocals (f < 2^23),
      // corrected
      int h = (int)((float)f * p.inv_run);
      if (h * run > f) --h;
      if ((h + 1) * run <= f) ++h;
      const int r = f - h * run;
      int g = (int)((float)r * p.inv_cpr);
      if (g * cpr > r) --g;
      if ((g + 1) * cpr <= r) ++g;
      const int c = r - g * cpr;
      const bool ok = f < nch && g < nvalid;
      const uint32_t row = (uint32_t)(((int64_t)g * p.x_ts[s] + (int64_t)h * D) * ES);
      buf_load<16>(rx, ok ? row + (uint32_t)(c * 16) : kOutOfRange, own[s][u]);
      yoff[s][u] = ok ? (uint32_t)(((int64_t)h * p.y_hs[s] + (int64_t)g * p.y_ts[s]) * ES +
                                   c * 16)
                      : kOutOfRange;
      col[s][u] = c * V;
      tok[s][u] = g;
      if (s < 2) {
        if constexpr (SPLIT) {
          // first part: elements c*V + half ... (or, for the straddling
          // chunk, the row's last V/2 elements); second part: 8 bytes on,
          // or the row's first V/2 elements
          uint32_t a, b;
          if (c < hc) {
            a = (uint32_t)((c * V + half) * ES);
            b = a + 8;
          } else if (c == hc) {
            a = (uint32_t)((D - V / 2) * ES);
            b = 0;
          } else {
            a = (uint32_t)((c * V - half) * ES);
            b = a + 8;
          }
          Words<8> pa, pb;
          buf_load<8>(rx, ok ? row + a : kOutOfRange, pa);
          buf_load<8>(rx, ok ? row + b : kOutOfRange, pb);
          par[s][u].w[0] = pa.w[0];
          par[s][u].w[1] = pa.w[1];
          par[s][u].w[2] = pb.w[0];
          par[s][u].w[3] = pb.w[1];
        } else {
          const int cp = c < hc ? c + hc : c - hc;
          buf_load<16>(rx, ok ? row + (uint32_t)(cp * 16) : kOutOfRange, par[s][u]);
        }
      }
    }
  }

  // 3. The group's cos/sin, one (token, column) per thread, through LDS.
  if (tid < ncs) {
    float c, sn;
    if (p.cs_cache != nullptr && (uint32_t)pp < (uint32_t)p.cache_rows) {
      cached_cos_sin(p.cs_cache, (int64_t)pp * p.n_freq + tab.fidx[cj], c, sn);
    } else {
      angle_cos_sin(pp, inv, c, sn);
    }
    cs[cg * half + cj] = make_float2(c, sn);
  }
  __syncthreads();

  // 4. Rotate q and k, copy v, store in output order.
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int H = p.heads[s];
    const __amdgpu_buffer_rsrc_t ry = buffer_of(
        static_cast<const char*>(p.y[s]) + t0 * p.y_ts[s] * ES,
        H > 0 ? (uint32_t)(((int64_t)(G - 1) * p.y_ts[s] + (int64_t)(H - 1) * p.y_hs[s] + D) *
                           ES)
              : 0u);
#pragma unroll
    for (int u = 0; u < kPlanesTasks; ++u) {
      Words<16> out = own[s][u];
      if (s < 2 && yoff[s][u] != kOutOfRange) {
        float a[V], b[V];
        unpack<BF16, V>(own[s][u], a);
        unpack<BF16, V>(par[s][u], b);
        const float2* row_cs = cs + tok[s][u] * half;
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int e = col[s][u] + i;
          const bool second = e >= half;
          const float2 w = row_cs[second ? e - half : e];
          if constexpr (PREC == MROPE_PRECISION_EXACT) {
            const double pr = (double)b[i] * (double)w.y;
            a[i] = (float)__builtin_fma((double)a[i], (double)w.x, second ? pr : -pr);
          } else {
#pragma clang fp contract(off)
            constexpr bool CAST = BF16 && PREC == MROPE_PRECISION_DTYPE;
            float cf = w.x, sf = w.y;
            if constexpr (CAST) {
              cf = round_bf16(cf);
              sf = round_bf16(sf);
            }
            float po = a[i] * cf;
            float pq = b[i] * sf;
            if constexpr (CAST) {
              po = round_bf16(po);
              pq = round_bf16(pq);
            }
            a[i] = second ? po + pq : po - pq;
          }
        }
        pack<BF16, V>(a, out);
      }
      buf_store<BF16, 16, MROPE_PLANES_NT_STORES>(ry, yoff[s][u], out);
    }
  }
}

template <bool BF16, int PREC>
int launch_planes_t(QKParams p, const ColTable& tab, bool split, hipStream_t st) {
  fit_axis_rule(tab, p.half, p);
  const int64_t blocks = (p.T + p.nt - 1) / p.nt;
  const size_t lds = (size_t)p.nt * p.half * sizeof(float2);
  if (split)
    hipLaunchKernelGGL((planes_kernel<BF16, PREC, true>), dim3((unsigned)blocks),
                       dim3(kPlanesThreads), lds, st, p, tab);
  else
    hipLaunchKernelGGL((planes_kernel<BF16, PREC, false>), dim3((unsigned)blocks),
                       dim3(kPlanesThreads), lds, st, p, tab);
  return (int)hipGetLastError();
}

}  // namespace

int planes_max_chunks_per_tensor() { return kPlanesThreads * kPlanesTasks; }
int planes_max_cos_sin() { return kPlanesThreads; }

int launch_planes(int dtype, int prec, const QKParams& p, const ColTable& tab, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int es = dtype == MROPE_DTYPE_BF16 ? 2 : 4;
  const bool split = (p.half % (16 / es)) != 0;
  if (dtype == MROPE_DTYPE_BF16) {
    switch (prec) {
      case MROPE_PRECISION_EXACT: return launch_planes_t<true, MROPE_PRECISION_EXACT>(p, tab, split, st);
      case MROPE_PRECISION_DTYPE: return launch_planes_t<true, MROPE_PRECISION_DTYPE>(p, tab, split, st);
      case MROPE_PRECISION_FP32: return launch_planes_t<true, MROPE_PRECISION_FP32>(p, tab, split, st);
    }
  } else {
    switch (prec) {
      case MROPE_PRECISION_EXACT: return launch_planes_t<false, MROPE_PRECISION_EXACT>(p, tab, split, st);
      case MROPE_PRECISION_DTYPE: return launch_planes_t<false, MROPE_PRECISION_DTYPE>(p, tab, split, st);
    }
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace mrope
