// The flat q/k kernel for gfx950: the positions path without RMSNorm for
// rows that are not whole 256-byte line pairs (such as the vision tower's
// 72-wide heads), token-major or in per-head planes.  The arithmetic per
// element is qk_kernel's (mrope_kernels.hip), so the results are
// bit-identical.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mrope_device.h"

namespace mrope {
namespace {

// ---------------------------------------------------------------------------
// The flat q/k kernel (no RMSNorm, cos/sin from positions).  One wavefront
// per token, as in qk_kernel, but the token's block of heads*D elements of a
// tensor is read as consecutive V-element chunks, lane after lane: every load
// instruction covers 64 consecutive chunks whatever the row length.  (The
// per-row mapping of qk_kernel makes rows of 288 bytes straddle cache lines
// in every instruction.)  A rotary chunk's partner -- half/V chunks away in
// the same row -- is loaded by the same lane, and all loads of a batch of
// kFlatSteps x 64 chunks are issued before any of its stores.  The
// arithmetic per element is qk_kernel's, so the results are bit-identical.
// ---------------------------------------------------------------------------

constexpr int kFlatSteps = 6;
static_assert(kFlatSteps * kWaveSize == kFlatBatchChunks, "one batch of the flat kernel");

template <bool BF16, int V, int PREC, bool NTS>
__global__ void __launch_bounds__(kBlockThreads) flat_kernel(const QKParams p, const ColTable tab) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int CB = ES * V;
  extern __shared__ double lds[];
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int half = p.half;
  float* lc = reinterpret_cast<float*>(lds) + wib * 2 * half;   // binary32 cos/sin
  float* ls = lc + half;
  const int64_t t0 = (int64_t)blockIdx.x * kWavesPerBlock + wib;
  if (t0 >= p.T) return;

  for (int j = lane; j < half; j += kWaveSize) {
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
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int cpr = p.D / V;        // chunks per head row
  const int hc = half / V;        // chunks per rotary half
  const int rc = p.rd / V;        // rotary chunks per row
#pragma unroll 1
  for (int s = 0; s < kSlots; ++s) {
    const int H = p.heads[s];
    if (H == 0) continue;
    const bool rotate = s < 2;    // the third tensor (v) is copied
    const int nch = H * cpr;
    const __amdgpu_buffer_rsrc_t rx = buffer_of(
        static_cast<const char*>(p.x[s]) + t0 * p.x_ts[s] * ES, (uint32_t)(nch * CB));
    const __amdgpu_buffer_rsrc_t ry = buffer_of(
        static_cast<const char*>(p.y[s]) + t0 * p.y_ts[s] * ES,
        (uint32_t)(((int64_t)(H - 1) * p.y_hs[s] + p.D) * ES));
#pragma unroll 1
    for (int base = 0; base < nch; base += kWaveSize * kFlatSteps) {
      Words<CB> own[kFlatSteps], par[kFlatSteps];
      uint32_t yoff[kFlatSteps];
      int col[kFlatSteps];
      int kind[kFlatSteps];   // 0 first rotary half, 1 second half, 2 pass-through
#pragma unroll
      for (int u = 0; u < kFlatSteps; ++u) {
        const int f = base + u * kWaveSize + lane;
        const bool ok = f < nch;
        // row = f / cpr through a binary32 reciprocal (f < 2^23), corrected
        int row = (int)((float)f * p.inv_cpr);
        if (row * cpr > f) --row;
        if ((row + 1) * cpr <= f) ++row;
        const int c = f - row * cpr;
        int k, fp;
        if (!rotate || c >= rc) {
          k = 2;
          fp = f;
        } else if (c < hc) {
          k = 0;
          fp = f + hc;
        } else {
          k = 1;
          fp = f - hc;
        }
        kind[u] = k;
        col[u] = ok && k < 2 ? (k == 1 ? c - hc : c) * V : 0;
        buf_load<CB>(rx, ok ? (uint32_t)(f * CB) : kOutOfRange, own[u]);
        buf_load<CB>(rx, ok && k < 2 ? (uint32_t)(fp * CB) : kOutOfRange, par[u]);
        yoff[u] = ok ? (uint32_t)(((int64_t)row * p.y_hs[s] + (int64_t)c * V) * ES)
                     : kOutOfRange;
      }
#pragma unroll
      for (int u = 0; u < kFlatSteps; ++u) {
        Words<CB> out = own[u];
        if (kind[u] < 2) {
          float a[V], b[V];
          unpack<BF16, V>(own[u], a);
          unpack<BF16, V>(par[u], b);
          const float* cc = lc + col[u];
          const float* sc = ls + col[u];
          if constexpr (PREC == MROPE_PRECISION_EXACT) {
            const double sg = kind[u] == 0 ? -1.0 : 1.0;
#pragma unroll
            for (int i = 0; i < V; ++i)
              a[i] = (float)__builtin_fma((double)a[i], (double)cc[i],
                                          sg * ((double)b[i] * (double)sc[i]));
          } else {
#pragma clang fp contract(off)
            constexpr bool CAST = BF16 && PREC == MROPE_PRECISION_DTYPE;
#pragma unroll
            for (int i = 0; i < V; ++i) {
              float cf = (float)cc[i], sf = (float)sc[i];
              if constexpr (CAST) {
                cf = round_bf16(cf);
                sf = round_bf16(sf);
              }
              float po = a[i] * cf;
              float pp = b[i] * sf;
              if constexpr (CAST) {
                po = round_bf16(po);
                pp = round_bf16(pp);
              }
              a[i] = kind[u] == 0 ? po - pp : po + pp;
            }
          }
          pack<BF16, V>(a, out);
        }
        buf_store<BF16, CB, NTS>(ry, yoff[u], out);
      }
    }
  }
}

template <bool BF16, int V, int PREC>
int launch_flat_t(const QKParams& p, const ColTable& tab, hipStream_t st) {
  const int64_t blocks = (p.T + kWavesPerBlock - 1) / kWavesPerBlock;
  int lds = kWavesPerBlock * 2 * p.half * (int)sizeof(float);
  if (p.waves_cap > 0) {
    const int cap_lds = (kLdsPerCu / p.waves_cap) & ~511;
    if (cap_lds > lds) lds = cap_lds;
  }
  // Store policy.  bf16: non-temporal.  fp32: non-temporal when every output
  // is token-major (a wavefront's stores then cover whole lines: vision_2d
  // 105.4 -> 98.6 us), cached for per-head planes (a 288-byte row starts
  // mid-line on every other token, and non-temporal partial lines cost:
  // 175 -> 208 us).
  bool token_major = true;
  for (int s = 0; s < kSlots; ++s)
    if (p.heads[s] > 0 && p.y_hs[s] != p.D) token_major = false;
  if (BF16 ? MROPE_NT_STORES_BF16 : token_major)
    hipLaunchKernelGGL((flat_kernel<BF16, V, PREC, true>), dim3((unsigned)blocks),
                       dim3(kBlockThreads), lds, st, p, tab);
  else
    hipLaunchKernelGGL((flat_kernel<BF16, V, PREC, false>), dim3((unsigned)blocks),
                       dim3(kBlockThreads), lds, st, p, tab);
  return (int)hipGetLastError();
}

template <bool BF16, int V>
int launch_flat_v(int prec, const QKParams& p, const ColTable& tab, hipStream_t st) {
  switch (prec) {
    case MROPE_PRECISION_EXACT: return launch_flat_t<BF16, V, MROPE_PRECISION_EXACT>(p, tab, st);
    case MROPE_PRECISION_DTYPE: return launch_flat_t<BF16, V, MROPE_PRECISION_DTYPE>(p, tab, st);
    case MROPE_PRECISION_FP32:
      if constexpr (BF16) return launch_flat_t<BF16, V, MROPE_PRECISION_FP32>(p, tab, st);
      break;
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_flat(int dtype, int vec, int prec, const QKParams& p, const ColTable& tab,
                void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == MROPE_DTYPE_BF16) {
    switch (vec) {
      case 8: return launch_flat_v<true, 8>(prec, p, tab, st);
      case 4: return launch_flat_v<true, 4>(prec, p, tab, st);
      case 2: return launch_flat_v<true, 2>(prec, p, tab, st);
      case 1: return launch_flat_v<true, 1>(prec, p, tab, st);
    }
  } else {
    switch (vec) {
      case 4: return launch_flat_v<false, 4>(prec, p, tab, st);
      case 2: return launch_flat_v<false, 2>(prec, p, tab, st);
      case 1: return launch_flat_v<false, 1>(prec, p, tab, st);
    }
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace mrope
