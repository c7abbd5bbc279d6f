// Device helpers shared by the q/k kernels (mrope_kernels.hip,
// mrope_pipe.hip): chunk storage and bf16 packing, the rounding helpers, the
// float64 cross-lane sum, the binary32 reciprocal square root and sincos,
// raw buffer loads and stores, and the host-side fit of the axis table to a
// rule.  Everything sits in an unnamed namespace: each translation unit
// keeps its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mrope_internal.h"

// Non-temporal (streaming) hint on the row stores of qk_kernel and
// stage_kernel, by element type (flat_kernel chooses by output layout).
#ifndef MROPE_NT_STORES_BF16
#define MROPE_NT_STORES_BF16 1
#endif
#ifndef MROPE_NT_STORES_F32
#define MROPE_NT_STORES_F32 0
#endif

namespace mrope {
namespace {
constexpr int kLdsPerCu = 160 * 1024;

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

// Round a binary32 value to bfloat16, kept as binary32: converting the pair
// (0, x) puts bf16(x) in the high half over a zero low half, which is the
// binary32 pattern of bf16(x) -- one v_cvt_pk_bf16_f32, no unpacking.
__device__ __forceinline__ float round_bf16(float x) {
  return __builtin_bit_cast(float, pack_bf16(0.0f, x));
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
#pragma unroll
  for (int i = 0; i < V; ++i) {
    a[i] = round_bf16(a[i]);
    b[i] = round_bf16(b[i]);
  }
}

// The rotation as tensor operations on one lane's pairs (x1 = a[i],
// x2 = b[i]): out1 = x1*c - x2*s, out2 = x2*c + x1*s with every product and
// sum rounded to binary32 and no product fused into a sum.  CAST rounds
// cos/sin and both products to bfloat16 as well (bf16 tensor arithmetic
// with cos/sin cast to the tensor's dtype); the last rounding to the stored
// dtype happens when the chunk is packed.
template <bool CAST, int V>
__device__ __forceinline__ void rotate_tensor_ops(float (&a)[V], float (&b)[V],
                                                  const double (&ca)[V], const double (&sa)[V],
                                                  const double (&cb)[V], const double (&sb)[V]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < V; ++i) {
    float c1 = (float)ca[i], s1 = (float)sa[i];
    float c2 = (float)cb[i], s2 = (float)sb[i];
    if constexpr (CAST) {
      c1 = round_bf16(c1);
      s1 = round_bf16(s1);
      c2 = round_bf16(c2);
      s2 = round_bf16(s2);
    }
    float p1 = a[i] * c1;
    float p2 = b[i] * s1;
    float p3 = b[i] * c2;
    float p4 = a[i] * s2;
    if constexpr (CAST) {
      p1 = round_bf16(p1);
      p2 = round_bf16(p2);
      p3 = round_bf16(p3);
      p4 = round_bf16(p4);
    }
    a[i] = p1 - p2;
    b[i] = p3 + p4;
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
  // Every lane of these patterns reads an active lane, so no fill value is
  // needed (bound_ctrl set).
  lo = __builtin_amdgcn_mov_dpp(lo, CTRL, 0xF, 0xF, true);
  hi = __builtin_amdgcn_mov_dpp(hi, CTRL, 0xF, 0xF, true);
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

// (cos, sin) from a cache by position, at cache[2 * idx].  The empty asm
// uses the loaded values inside the caller's branch, so the compiler waits
// for this load there.  Left pending past the branch, it would make the
// compiler wait for every vector load in flight where the branches join,
// the row loads already issued included.
__device__ __forceinline__ void cached_cos_sin(const float* cache, int64_t idx, float& c,
                                               float& s) {
  const float2 cs = *reinterpret_cast<const float2*>(cache + 2 * idx);
  c = cs.x;
  s = cs.y;
  asm volatile("" : : "v"(c), "v"(s));
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

// Cross-lane float64 sum over the LPR lanes of a row (LPR a power of two
// known at compile time), or over p.lpr lanes when LPR == 0.
template <int LPR>
__device__ __forceinline__ double row_sum(double v, int lpr) {
  if constexpr (LPR == 0) {
    return group_sum(v, lpr);
  } else {
    if constexpr (LPR >= 2) v += dpp_f64<0xB1>(v);
    if constexpr (LPR >= 4) v += dpp_f64<0x4E>(v);
    if constexpr (LPR >= 8) v += dpp_f64<0x141>(v);
    if constexpr (LPR >= 16) v += dpp_f64<0x140>(v);
    if constexpr (LPR >= 32) v += __shfl_xor(v, 16);
    if constexpr (LPR >= 64) v += __shfl_xor(v, 32);
    return v;
  }
}

// Raw buffer access.  A descriptor covers one tile of one tensor; an offset
// past its range makes a load return zeros and drops a store in hardware, so
// masked rows issue the same instructions as live ones with no branch around
// them (which also keeps the compiler's memory-counter waits exact).
constexpr int kBufferWord3 = 0x00020000;    // gfx9 raw buffer, dword data
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferWord3);
}

// NT: non-temporal (streaming) load, aux 2, for data the kernel reads
// exactly once: the caches keep its lines at the lowest priority.
template <int CB, bool NT = false>
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t rs, uint32_t off, Words<CB>& r) {
  constexpr int aux = NT ? 2 : 0;
  if constexpr (CB == 16) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, aux);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (CB == 8) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, aux);
    r.w[0] = v.x; r.w[1] = v.y;
  } else if constexpr (CB == 4) {
    r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, aux);
  } else {
    r.w[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, aux);
  }
}

// NT: non-temporal (streaming) store, aux 2.  The default is measured per
// dtype for qk_kernel and stage_kernel; flat_kernel chooses by output layout.
template <bool BF16, int CB, bool NT = (BF16 ? MROPE_NT_STORES_BF16 : MROPE_NT_STORES_F32)>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                          const Words<CB>& r) {
  constexpr int aux = NT ? 2 : 0;
  if constexpr (CB == 16) {
    const u32x4_t v = {r.w[0], r.w[1], r.w[2], r.w[3]};
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, aux);
  } else if constexpr (CB == 8) {
    const u32x2_t v = {r.w[0], r.w[1]};
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, aux);
  } else if constexpr (CB == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(r.w[0], rs, off, 0, aux);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)r.w[0], rs, off, 0, aux);
  }
}

// The axis table as one of the kernel's two rules (ax_mode 0 or 1), or -1.
inline void fit_axis_rule(const ColTable& tab, int half, QKParams& p) {
  int n0 = 0, n1 = 0, n2 = 0;
  bool sorted = true;
  for (int j = 0; j < half; ++j) {
    n0 += tab.axis[j] == 0;
    n1 += tab.axis[j] == 1;
    n2 += tab.axis[j] == 2;
    if (j > 0 && tab.axis[j] < tab.axis[j - 1]) sorted = false;
  }
  for (int mode = 0; mode < 2; ++mode) {
    const int a = mode == 0 ? n0 : 3 * n1;
    const int b = mode == 0 ? n0 + n1 : 3 * n2;
    if (mode == 0 && !sorted) continue;
    bool ok = true;
    for (int j = 0; j < half && ok; ++j) {
      const int ax = mode == 0 ? (j >= a) + (j >= b)
                              : (j % 3 == 1 && j < a) ? 1 : (j % 3 == 2 && j < b) ? 2 : 0;
      ok = ax == tab.axis[j];
    }
    if (ok) {
      p.ax_mode = mode;
      p.ax_a = a;
      p.ax_b = b;
      return;
    }
  }
  p.ax_mode = -1;
  p.ax_a = p.ax_b = 0;
}

}  // namespace
}  // namespace mrope
