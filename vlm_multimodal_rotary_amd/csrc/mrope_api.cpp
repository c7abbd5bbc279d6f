// C-ABI entry points: argument checking, the per-column frequency/axis table,
// launch geometry, and the kernel launches.  Every check runs before the first
// HIP call, so an invalid call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "mrope_internal.h"

namespace {

thread_local std::string g_err;
thread_local const char* g_last_kernel = "";

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MROPE_OK;
}

// Byte extent of a [T][heads][D] view with the given token stride.
struct Extent {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  bool empty() const { return hi <= lo; }
};

Extent extent_of(const void* base, int64_t T, int64_t tok_stride, int64_t row_elems,
                 int elem_bytes) {
  Extent e;
  if (base == nullptr || T <= 0 || row_elems <= 0) return e;
  e.lo = reinterpret_cast<uintptr_t>(base);
  e.hi = e.lo + (uintptr_t)(((T - 1) * tok_stride + row_elems) * elem_bytes);
  return e;
}

bool overlaps(const Extent& a, const Extent& b) {
  if (a.empty() || b.empty()) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// An output may equal its own input exactly (same base and stride); any other
// overlap is rejected.
bool bad_alias(const Extent& out, const Extent& in, bool same_view) {
  return overlaps(out, in) && !same_view;
}

int elem_bytes_of(int dtype) { return dtype == MROPE_DTYPE_BF16 ? 2 : 4; }

int check_dtype(int dtype) {
  if (dtype != MROPE_DTYPE_F32 && dtype != MROPE_DTYPE_BF16)
    return fail(MROPE_EUNSUPPORTED, "dtype %d is not MROPE_DTYPE_F32 (0) or MROPE_DTYPE_BF16 (1)",
                dtype);
  return MROPE_OK;
}

// inv[i] = theta^(-2i/dim), double evaluation rounded once.  The values of
// the calling thread's last (dim, theta) are kept: the layers of a model call
// with the same pair, and the pow calls are the largest part of the host work
// of a small launch.
void fill_inv(int dim, double theta, float* out) {
  thread_local int last_dim = 0;
  thread_local double last_theta = 0.0;
  thread_local float last[mrope::kMaxHalf];
  const int n = dim / 2;
  if (n > 0 && n <= mrope::kMaxHalf && dim == last_dim && theta == last_theta) {
    std::memcpy(out, last, sizeof(float) * (size_t)n);
    return;
  }
  for (int i = 0; i < n; ++i) out[i] = (float)std::pow(theta, -(2.0 * i) / (double)dim);
  if (n > 0 && n <= mrope::kMaxHalf) {
    std::memcpy(last, out, sizeof(float) * (size_t)n);
    last_dim = dim;
    last_theta = theta;
  }
}

int build_axis(int half, const int* section, int n_sections, int layout, uint8_t* axis) {
  if (half <= 0 || half > mrope::kMaxHalf)
    return fail(MROPE_EINVAL, "half = %d outside [1, %d]", half, mrope::kMaxHalf);
  if (layout == MROPE_LAYOUT_VISION_2D) {
    if (half % 2 != 0) return fail(MROPE_EINVAL, "vision layout needs an even half, got %d", half);
    for (int j = 0; j < half; ++j) axis[j] = (uint8_t)(j < half / 2 ? 0 : 1);
    return MROPE_OK;
  }
  if (layout != MROPE_LAYOUT_CHUNKED && layout != MROPE_LAYOUT_INTERLEAVED)
    return fail(MROPE_EINVAL, "unknown layout %d", layout);
  if (section == nullptr) return fail(MROPE_EINVAL, "section is NULL");
  if (layout == MROPE_LAYOUT_INTERLEAVED && n_sections != 3)
    return fail(MROPE_EINVAL, "interleaved layout needs 3 section entries, got %d", n_sections);
  if (n_sections < 1 || n_sections > 3)
    return fail(MROPE_EINVAL, "chunked layout needs 1..3 section entries, got %d", n_sections);
  int sum = 0;
  for (int a = 0; a < n_sections; ++a) {
    if (section[a] < 0) return fail(MROPE_EINVAL, "section[%d] = %d is negative", a, section[a]);
    sum += section[a];
  }
  if (sum != half)
    return fail(MROPE_EINVAL, "section sums to %d, rotary_dim/2 is %d", sum, half);
  if (layout == MROPE_LAYOUT_CHUNKED) {
    int j = 0;
    for (int a = 0; a < n_sections; ++a)
      for (int c = 0; c < section[a]; ++c) axis[j++] = (uint8_t)a;
    return MROPE_OK;
  }
  // Interleaved: H on j % 3 == 1 below 3*s_h, W on j % 3 == 2 below 3*s_w,
  // T elsewhere.  The rule places every H and W column only if the last one
  // falls inside [0, half).
  const int sh = section[1], sw = section[2];
  if (sh > 0 && 3 * (sh - 1) + 1 >= half)
    return fail(MROPE_EINVAL, "interleaved section [%d,%d,%d]: H column %d is past half = %d",
                section[0], sh, sw, 3 * (sh - 1) + 1, half);
  if (sw > 0 && 3 * (sw - 1) + 2 >= half)
    return fail(MROPE_EINVAL, "interleaved section [%d,%d,%d]: W column %d is past half = %d",
                section[0], sh, sw, 3 * (sw - 1) + 2, half);
  for (int j = 0; j < half; ++j) {
    uint8_t a = 0;
    if (j % 3 == 1 && j < 3 * sh) a = 1;
    else if (j % 3 == 2 && j < 3 * sw) a = 2;
    axis[j] = a;
  }
  return MROPE_OK;
}

int expected_axes(int layout, int n_sections) {
  if (layout == MROPE_LAYOUT_INTERLEAVED) return 3;
  if (layout == MROPE_LAYOUT_VISION_2D) return 2;
  return n_sections;
}

// Column table of the fused path: inverse frequency per column and its axis.
int build_table(int rotary_dim, double theta, const int* section, int n_sections, int layout,
                const float* inv_given, mrope::ColTable& tab) {
  const int half = rotary_dim / 2;
  int rc = build_axis(half, section, n_sections, layout, tab.axis);
  if (rc) return rc;
  for (int j = 0; j < half; ++j)
    tab.fidx[j] = (uint8_t)(layout == MROPE_LAYOUT_VISION_2D ? j % (half / 2) : j);
  if (inv_given != nullptr) {
    for (int j = 0; j < half; ++j)
      tab.inv[j] = layout == MROPE_LAYOUT_VISION_2D ? inv_given[j % (half / 2)] : inv_given[j];
    return MROPE_OK;
  }
  if (layout == MROPE_LAYOUT_VISION_2D) {
    float inv[mrope::kMaxHalf / 2];
    fill_inv(half, theta, inv);
    for (int j = 0; j < half; ++j) tab.inv[j] = inv[j % (half / 2)];
  } else {
    fill_inv(rotary_dim, theta, tab.inv);
  }
  return MROPE_OK;
}

// Largest chunk (elements) that keeps every access aligned and the lane
// mapping exact: rotary chunks tile [0, half), pass-through lanes own two
// chunks of [rd, D).
int pick_vec(int dtype, int D, int rd, const void* const* ptrs, int nptrs,
             const int64_t* strides, int nstrides) {
  const int es = elem_bytes_of(dtype);
  const int max_v = 16 / es;
  const int half = rd / 2;
  for (int v = max_v; v >= 1; v /= 2) {
    if (D % (2 * v) != 0) continue;
    if (half % v != 0) continue;
    if ((D - rd) % (2 * v) != 0) continue;
    if (D / (2 * v) > mrope::kWaveSize) continue;
    bool good = true;
    for (int i = 0; i < nptrs && good; ++i)
      if (ptrs[i] != nullptr && (reinterpret_cast<uintptr_t>(ptrs[i]) % (uintptr_t)(v * es)) != 0)
        good = false;
    for (int i = 0; i < nstrides && good; ++i)
      if (strides[i] % v != 0) good = false;
    if (good) return v;
  }
  return 0;
}

// Up to three tensors (q, k, and the v of a packed qkv that is only copied).
// Inputs have contiguous heads (head stride D); outputs have a head stride
// (0 = D, token-major rows).
constexpr int kSlots = mrope::kSlots;
constexpr int64_t kFlatMinTokens = 2048;   // one wavefront per token fills the chip
constexpr int kMaxHeads = 1 << 20;          // heads per tensor
constexpr int64_t kFlatMaxChunks = 1 << 22; // chunks of one token's rows in the flat kernel
constexpr int kStageLdsTarget = 32 * 1024;  // LDS of a staged block: five or more per CU
constexpr int kStageLdsMax = 64 * 1024;     // ... at most (two per CU), with G forced

struct QKArgs {
  const void* x[kSlots];
  int64_t x_ts[kSlots];
  int heads[kSlots];
  void* y[kSlots];
  int64_t y_ts[kSlots];
  int64_t y_hs[kSlots];
  const void* w[kSlots];
  int64_t T;
  int D, rd, dtype;
  int precision;  // MROPE_PRECISION_*; EXACT for RMSNorm only
};

int64_t head_stride(const QKArgs& a, int s) { return a.y_hs[s] != 0 ? a.y_hs[s] : a.D; }

// Byte extent of an output [T][H][D] view with token and head strides.
Extent out_extent(const QKArgs& a, int s, int es) {
  Extent e;
  if (a.y[s] == nullptr || a.T <= 0 || a.heads[s] <= 0) return e;
  e.lo = reinterpret_cast<uintptr_t>(a.y[s]);
  e.hi = e.lo + (uintptr_t)(((a.T - 1) * a.y_ts[s] + (int64_t)(a.heads[s] - 1) * head_stride(a, s) +
                             a.D) * es);
  return e;
}

int check_qk_tensors(const QKArgs& a, bool need_rd) {
  int rc = check_dtype(a.dtype);
  if (rc) return rc;
  if (a.precision != MROPE_PRECISION_EXACT && a.precision != MROPE_PRECISION_DTYPE &&
      a.precision != MROPE_PRECISION_FP32)
    return fail(MROPE_EINVAL, "precision %d is not one of MROPE_PRECISION_EXACT (0), "
                "_DTYPE (1) or _FP32 (2)", a.precision);
  if (a.T < 0) return fail(MROPE_EINVAL, "T = %lld is negative", (long long)a.T);
  if (a.D <= 0 || a.D % 2 != 0) return fail(MROPE_EINVAL, "D = %d must be positive and even", a.D);
  if (need_rd) {
    if (a.rd <= 0 || a.rd % 2 != 0 || a.rd > a.D)
      return fail(MROPE_EINVAL, "rotary_dim = %d must be even, positive and <= D = %d", a.rd, a.D);
    if (a.rd > MROPE_MAX_ROTARY_DIM)
      return fail(MROPE_EUNSUPPORTED, "rotary_dim = %d exceeds %d", a.rd, MROPE_MAX_ROTARY_DIM);
  }
  const char* nm[kSlots] = {"q", "k", "v"};
  for (int s = 0; s < kSlots; ++s) {
    if (a.heads[s] < 0) return fail(MROPE_EINVAL, "%s heads = %d is negative", nm[s], a.heads[s]);
    // the kernels split row indices through binary32 reciprocals, exact for
    // the index ranges this bound keeps
    if (a.heads[s] > kMaxHeads)
      return fail(MROPE_EUNSUPPORTED, "%s heads = %d exceed %d", nm[s], a.heads[s], kMaxHeads);
    if (a.heads[s] == 0 || a.T == 0) continue;
    if (a.x[s] == nullptr) return fail(MROPE_EINVAL, "%s input is NULL", nm[s]);
    if (a.y[s] == nullptr) return fail(MROPE_EINVAL, "%s output is NULL", nm[s]);
    const int64_t row = (int64_t)a.heads[s] * a.D;
    if (a.x_ts[s] < row)
      return fail(MROPE_EINVAL, "%s token stride %lld < heads*D = %lld", nm[s],
                  (long long)a.x_ts[s], (long long)row);
    // output rows must not overlap one another: heads inside tokens
    // (token-major) or tokens inside heads (head-major planes)
    const int64_t hs = head_stride(a, s);
    const bool token_major = hs >= a.D && a.y_ts[s] >= (int64_t)a.heads[s] * hs;
    const bool head_major = a.y_ts[s] >= a.D && (a.heads[s] == 1 || hs >= a.T * a.y_ts[s]);
    if (!token_major && !head_major)
      return fail(MROPE_EINVAL, "%s output strides (token %lld, head %lld) overlap rows of "
                  "heads*D = %lld", nm[s], (long long)a.y_ts[s], (long long)hs, (long long)row);
  }
  // Overlap rules.
  const int es = elem_bytes_of(a.dtype);
  Extent xin[kSlots], yout[kSlots];
  for (int s = 0; s < kSlots; ++s) {
    const bool live = a.heads[s] > 0 && a.T > 0;
    const int64_t row = (int64_t)a.heads[s] * a.D;
    if (live) {
      xin[s] = extent_of(a.x[s], a.T, a.x_ts[s], row, es);
      yout[s] = out_extent(a, s, es);
    }
  }
  for (int s = 0; s < kSlots; ++s) {
    const bool same = a.x[s] == a.y[s] && a.x_ts[s] == a.y_ts[s] && head_stride(a, s) == a.D;
    if (bad_alias(yout[s], xin[s], same))
      return fail(MROPE_EINVAL, "%s output partially overlaps its input", nm[s]);
    for (int o = 0; o < kSlots; ++o) {
      if (o == s) continue;
      if (overlaps(yout[s], xin[o]))
        return fail(MROPE_EINVAL, "%s output overlaps the %s input", nm[s], nm[o]);
      if (o > s && overlaps(yout[s], yout[o]))
        return fail(MROPE_EINVAL, "%s and %s outputs overlap", nm[s], nm[o]);
    }
  }
  for (int s = 0; s < kSlots; ++s) {
    if (a.w[s] == nullptr) continue;
    Extent we = extent_of(a.w[s], 1, a.D, a.D, es);
    for (int o = 0; o < kSlots; ++o)
      if (overlaps(yout[o], we)) return fail(MROPE_EINVAL, "an output overlaps a weight vector");
  }
  return MROPE_OK;
}

// An optional cos/sin cache by position for the positions path.
struct CacheArgs {
  const float* cache = nullptr;
  int rows = 0;
  int n_freq = 0;
};

// Checks an optional cos/sin cache argument of the positions path: rows of
// n_freq (cos, sin) pairs, 8-byte aligned, not overlapping any output.
int check_cache(const float* cache, int rows, int n_freq, CacheArgs& out, Extent& ext) {
  out = CacheArgs();
  ext = Extent();
  if (cache == nullptr) {
    if (rows != 0) return fail(MROPE_EINVAL, "cache_rows must be 0 without a cache");
    return MROPE_OK;
  }
  if (rows < 0) return fail(MROPE_EINVAL, "cache_rows is negative");
  if (reinterpret_cast<uintptr_t>(cache) % 8 != 0)
    return fail(MROPE_EINVAL, "the cos/sin cache must be 8-byte aligned");
  ext = extent_of(cache, 1, 0, (int64_t)rows * n_freq * 2, 4);
  out.cache = cache;
  out.rows = rows;
  out.n_freq = n_freq;
  return MROPE_OK;
}

// Resident wavefronts per SIMD for a launch (0 = as many as registers allow).
// Measured on MI355X: per-head-plane outputs (many short scattered row
// writes per wavefront) run best with few wavefronts -- 3 for 8-byte chunks,
// 4 for 16-byte chunks; token-major launches with 16 lanes per head row or
// more (D >= 256 bf16) gain a little from 5; everything else runs unbounded.
// MROPE_WAVES_PER_SIMD in the environment overrides the choice (tuning).
int waves_per_simd(const QKArgs& a, int v, int es) {
  static const int env = [] {
    const char* e = std::getenv("MROPE_WAVES_PER_SIMD");
    return e != nullptr ? std::atoi(e) : -1;
  }();
  if (env >= 0) return env > 8 ? 8 : env;
  bool planes = false;
  for (int s = 0; s < kSlots; ++s)
    if (a.heads[s] > 0 && head_stride(a, s) != a.D) planes = true;
  const int chunk_bytes = v * es;
  if (planes) return chunk_bytes < 16 ? 3 : 4;
  if (a.D / (2 * v) >= 16 && chunk_bytes == 16 && es == 2) return 5;
  return 0;
}

int env_int(const char* name, int fallback) {
  const char* e = std::getenv(name);
  return e != nullptr ? std::atoi(e) : fallback;
}

// The flat kernel (chunks of the token's block lane after lane) serves the
// positions path without RMSNorm for launches of at least one wavefront per
// token over the whole chip.  It is chosen where the per-row mapping leaves
// rows straddling cache lines (row bytes not a multiple of 256).  An
// in-place tensor qualifies only if a token's rows fit one load batch (the
// kernel stores a batch before it loads the next, and a rotary partner may
// sit in the next batch).  MROPE_FLAT=0/1 in the environment forces the
// choice where it is allowed (tuning).
bool use_flat(const QKArgs& a, int cs_mode, bool norm, int v, int es) {
  if (cs_mode != mrope::kCsFromPositions || norm || a.T < kFlatMinTokens) return false;
  for (int s = 0; s < kSlots; ++s) {
    const int64_t chunks = (int64_t)a.heads[s] * (a.D / v);
    // the row of a chunk comes from a binary32 reciprocal: exact below 2^22
    if (chunks >= kFlatMaxChunks) return false;
    if (a.heads[s] > 0 && a.x[s] == a.y[s] && chunks > mrope::kFlatBatchChunks) return false;
  }
  static const int env = env_int("MROPE_FLAT", -1);
  if (env >= 0) return env != 0;
  return (a.D * es) % 256 != 0;
}

// Resident wavefronts per SIMD for the flat kernel (0 = unbounded).  Four
// measured best on the 72-wide vision rows in f32 and bf16, token-major and
// head-major (two and three trail by 10%, unbounded by 1-10%).
int waves_per_simd_flat() {
  static const int env = env_int("MROPE_WAVES_PER_SIMD", -1);
  if (env >= 0) return env > 8 ? 8 : env;
  return 4;
}

// The staged kernel (q/k rows copied to LDS G tokens at a time, written back
// in output order; v through registers) serves the positions path without
// RMSNorm when every base, stride and row is 16-byte aligned and the rotary
// half is even.  It is chosen for bfloat16 head-major outputs (per-head
// planes), where it writes each head's G rows as one run: 74% of HBM peak on
// 16 x 72 bf16 planes against 51% for the flat kernel.  For binary32 planes
// and token-major rows the flat kernel measured faster (64% and 72% against
// 58% and 61%).  Every read of a block lands before its first write, so
// in-place calls are safe.
// Returns the largest G to try (the caller shrinks it to the LDS budget), or
// 0 for another kernel.  MROPE_STAGE=0/1 and MROPE_STAGE_G in the
// environment force the choice.
int pick_stage(const QKArgs& a, int cs_mode, bool norm, int es, bool& head_major) {
  if (cs_mode != mrope::kCsFromPositions || norm || a.T < kFlatMinTokens) return 0;
  if (a.rd <= 0 || (a.rd / 2) % 2 != 0 || (a.D * es) % 16 != 0) return 0;
  bool hm = false, tm = false;
  for (int s = 0; s < kSlots; ++s) {
    if (a.heads[s] == 0) continue;
    const int64_t hs = head_stride(a, s);
    if ((reinterpret_cast<uintptr_t>(a.x[s]) | reinterpret_cast<uintptr_t>(a.y[s])) % 16 != 0)
      return 0;
    if ((a.x_ts[s] * es) % 16 != 0 || (a.y_ts[s] * es) % 16 != 0 || (hs * es) % 16 != 0)
      return 0;
    if (hs == a.D && a.heads[s] > 1) tm = true;
    else hm = true;
  }
  if (hm && tm) return 0;
  head_major = hm;
  static const int env = env_int("MROPE_STAGE", -1);
  static const int env_g = env_int("MROPE_STAGE_G", 0);
  if (env == 0 || (env < 0 && !(hm && es == 2))) return 0;
  const int G = env_g > 0 ? env_g : 16;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return 0;
  // a block's rows of each tensor are addressed with 32-bit byte offsets
  const int64_t limit = int64_t(1) << 31;
  for (int s = 0; s < kSlots; ++s) {
    if (a.heads[s] == 0) continue;
    const int64_t H = a.heads[s];
    if (((G - 1) * a.x_ts[s] + H * a.D) * es >= limit ||
        ((G - 1) * a.y_ts[s] + (H - 1) * head_stride(a, s) + a.D) * es >= limit)
      return 0;
  }
  return G;
}

// Tokens per block of the group kernel (0: not taken).  It serves the
// positions path without RMSNorm with full rotary into per-head planes, on
// 16-byte aligned rows whose half is a multiple of half a chunk, out of
// place; the tokens per block (the fewest that make each plane's run of
// rows a whole number of 128-byte lines) must fit the block.  Measured on
// the vision tower's planes (16 heads of 72, 32768 patches, rotating
// buffer sets): fp32 177.0 -> 166.0 us against the flat kernel, bf16 97.6
// -> 93.5 us against the staged kernel.  MROPE_PLANES=0/1 and
// MROPE_PLANES_G force the choice (tuning).
int pick_planes(const QKArgs& a, int cs_mode, bool norm, int es) {
  static const int env = env_int("MROPE_PLANES", -1);
  static const int env_g = env_int("MROPE_PLANES_G", 0);
  if (env == 0) return 0;
  if (cs_mode != mrope::kCsFromPositions || norm || a.T < kFlatMinTokens) return 0;
  bool planes = true;
  for (int s = 0; s < kSlots; ++s)
    if (a.heads[s] > 0 && head_stride(a, s) == a.D) planes = false;
  if (!planes && env < 0) return 0;
  const int V = 16 / es;
  const int half = a.rd / 2;
  if (a.rd != a.D || (a.D * es) % 16 != 0 || (2 * half) % V != 0) return 0;
  for (int s = 0; s < kSlots; ++s) {
    if (a.heads[s] == 0) continue;
    if ((reinterpret_cast<uintptr_t>(a.x[s]) | reinterpret_cast<uintptr_t>(a.y[s])) % 16 != 0)
      return 0;
    if ((a.x_ts[s] * es) % 16 != 0 || (a.y_ts[s] * es) % 16 != 0 ||
        (head_stride(a, s) * es) % 16 != 0)
      return 0;
    // out of place only: a block's stores may land before another block's
    // loads of the same lines
    for (int s2 = 0; s2 < kSlots; ++s2) {
      if (a.heads[s2] == 0) continue;
      Extent in;
      in.lo = reinterpret_cast<uintptr_t>(a.x[s2]);
      in.hi = in.lo + (uintptr_t)(((a.T - 1) * a.x_ts[s2] + (int64_t)a.heads[s2] * a.D) * es);
      if (overlaps(in, out_extent(a, s, es))) return 0;
    }
  }
  int G = env_g > 0 ? env_g : 1;
  if (env_g <= 0)
    while (G < 16 && ((int64_t)G * a.D * es) % 128 != 0) G *= 2;
  const int cpr = a.D / V;
  auto fits = [&](int g) {
    if (g * half > mrope::planes_max_cos_sin()) return false;
    for (int s = 0; s < kSlots; ++s)
      if ((int64_t)a.heads[s] * g * cpr > mrope::planes_max_chunks_per_tensor()) return false;
    // a block's rows of each tensor are addressed with 32-bit byte offsets
    const int64_t limit = int64_t(1) << 31;
    for (int s = 0; s < kSlots; ++s) {
      if (a.heads[s] == 0) continue;
      const int64_t H = a.heads[s];
      if (((g - 1) * a.x_ts[s] + H * a.D) * es >= limit ||
          ((g - 1) * a.y_ts[s] + (H - 1) * head_stride(a, s) + a.D) * es >= limit)
        return false;
    }
    return true;
  };
  return fits(G) ? G : 0;
}

// Resident wavefronts per SIMD for the staged kernel (0 = as LDS allows).
int waves_per_simd_stage() {
  static const int env = env_int("MROPE_WAVES_PER_SIMD", -1);
  if (env >= 0) return env > 8 ? 8 : env;
  return 0;
}

// The pipelined q/k kernel (one token per wavefront, its row-steps as one
// stream with P steps of loads in flight while it finishes a step, cos/sin in
// registers) serves the positions path for 16-byte chunks when the launch has
// at least kMinPipeTokens tokens.  Measured on MI355X with inputs that the
// memory-side cache does not hold (rotating buffer sets), against qk_kernel.
// MROPE_PIPE=0/1 forces the choice where it is allowed (tuning).
constexpr int64_t kMinPipeTokens = 2048;

bool use_pipe(const QKArgs& a, int cs_mode, int v, int es) {
  if (cs_mode != mrope::kCsFromPositions || v * es != 16 || a.T < kMinPipeTokens) return false;
  static const int env = env_int("MROPE_PIPE", -1);
  if (env >= 0) return env != 0;
  return true;
}

// Launch geometry and the remaining per-launch fields.
struct DecodeArgs {
  const int32_t* cache_len = nullptr;
  const int32_t* rope_delta = nullptr;
  int new_tokens = 0;
  int64_t kc_seq = 0, kc_tok = 0;
  int kc_cap = 0;
};

int run_qk(const QKArgs& a, int cs_mode, bool norm, const mrope::ColTable& tab,
           const int32_t* pos, int64_t pos_stride, const float* cos, const float* sin,
           int64_t cs_ts, float eps, void* stream, const Extent* extra, int n_extra,
           const DecodeArgs* dec = nullptr, const CacheArgs* cache = nullptr) {
  const int es = elem_bytes_of(a.dtype);
  const void* ptrs[9] = {a.x[0], a.x[1], a.x[2], a.y[0], a.y[1], a.y[2], a.w[0], a.w[1], a.w[2]};
  int64_t strides[11] = {a.x_ts[0], a.x_ts[1], a.x_ts[2], a.y_ts[0], a.y_ts[1], a.y_ts[2],
                         head_stride(a, 0), head_stride(a, 1), head_stride(a, 2),
                         dec ? dec->kc_seq : 0, dec ? dec->kc_tok : 0};
  const int v = pick_vec(a.dtype, a.D, a.rd, ptrs, 9, strides, 11);
  if (v == 0)
    return fail(MROPE_EUNSUPPORTED,
                "no vector width fits D = %d, rotary_dim = %d and the buffer alignment "
                "(need element-aligned pointers and D/2 lanes or fewer per row)",
                a.D, a.rd);
  for (int i = 0; i < n_extra; ++i)
    for (int o = 0; o < kSlots; ++o)
      if (overlaps(out_extent(a, o, es), extra[i]))
        return fail(MROPE_EINVAL, "an output overlaps a positions or cos/sin buffer");
  if (a.T == 0 || a.heads[0] + a.heads[1] + a.heads[2] == 0) return ok();

  mrope::QKParams p;
  std::memset(&p, 0, sizeof(p));
  for (int s = 0; s < kSlots; ++s) {
    p.x[s] = a.x[s];
    p.y[s] = a.y[s];
    p.w[s] = a.w[s];
    p.y_hs[s] = head_stride(a, s);
    p.x_ts[s] = a.x_ts[s];
    p.y_ts[s] = a.y_ts[s];
    p.heads[s] = a.heads[s];
  }
  p.T = a.T;
  p.D = a.D;
  p.rd = a.rd;
  p.half = a.rd / 2;
  p.lpr = a.D / (2 * v);
  p.rpw = mrope::kWaveSize / p.lpr;
  p.lrot = p.half / v;
  p.pos = pos;
  p.pos_stride = pos_stride;
  p.cos = cos;
  p.sin = sin;
  p.cs_ts = cs_ts;
  p.eps = eps;
  p.inv_d = 1.0 / (double)a.D;
  if (cache != nullptr && cache->cache != nullptr) {
    p.cs_cache = cache->cache;
    p.cache_rows = cache->rows;
    p.n_freq = cache->n_freq;
  }
  if (dec != nullptr) {
    p.cache_len = dec->cache_len;
    p.rope_delta = dec->rope_delta;
    p.new_tokens = dec->new_tokens;
    p.kc_seq = dec->kc_seq;
    p.kc_tok = dec->kc_tok;
    p.kc_cap = dec->kc_cap;
  }

  // Tokens per tile: a wavefront's cos/sin slice (2 * nt * half binary32
  // values) stays within 4 KB.
  int nt_cap = p.half > 0 ? 512 / p.half : 16;
  if (nt_cap < 1) nt_cap = 1;
  if (nt_cap > 16) nt_cap = 16;
  // The kernels address a tile of each tensor through a buffer descriptor
  // with 32-bit byte offsets: a tile's extent must stay below 2^31 bytes.
  const int64_t limit = int64_t(1) << 31;
  for (int s = 0; s < kSlots; ++s) {
    if (a.heads[s] == 0) continue;
    const int64_t H = a.heads[s];
    auto in_ext = [&](int64_t nt) { return ((nt - 1) * a.x_ts[s] + H * a.D) * es; };
    auto out_ext = [&](int64_t nt) {
      return ((nt - 1) * a.y_ts[s] + (H - 1) * head_stride(a, s) + a.D) * es;
    };
    while (nt_cap > 1 && (in_ext(nt_cap) >= limit || out_ext(nt_cap) >= limit)) --nt_cap;
    if (in_ext(1) >= limit || out_ext(1) >= limit)
      return fail(MROPE_EUNSUPPORTED, "one token's rows of %s span 2^31 bytes or more",
                  s == 0 ? "q" : (s == 1 ? "k" : "v"));
  }
  // Tokens per wavefront.  With RMSNorm on the positions path: the fewest
  // tokens (1, 2 or 4) whose rows fill whole row-steps of every tensor, so
  // no lane group runs the norm's arithmetic on a masked row -- 4 k heads at
  // 8 rows per step take 2 tokens.  Measured on the 32 + 4 head bf16 prefill:
  // 107.2 -> 103.0 us; launches without the norm, whose rows already fill
  // their steps or that are bound by memory alone, ran slower with more
  // tokens per wavefront.  MROPE_WAVE_TOKENS in the environment forces the
  // count (tuning).
  {
    static const int env = env_int("MROPE_WAVE_TOKENS", 0);
    int wave_tokens = 1;
    if (env > 0) {
      wave_tokens = env;
    } else if (norm && cs_mode == mrope::kCsFromPositions) {
      for (int n = 1; n <= 4; n *= 2) {
        bool whole = true;
        for (int s = 0; s < kSlots; ++s)
          if (a.heads[s] > 0 && (n * a.heads[s]) % p.rpw != 0) whole = false;
        if (whole) {
          wave_tokens = n;
          break;
        }
      }
    }
    if (nt_cap > wave_tokens) nt_cap = wave_tokens;
  }
  // For binary32 tensors the cast of cos/sin to the dtype is the identity.
  const int prec = (a.dtype == MROPE_DTYPE_F32 && a.precision == MROPE_PRECISION_FP32)
                       ? MROPE_PRECISION_DTYPE : a.precision;
  int hrc;
  bool head_major = false;
  const int GP = pick_planes(a, cs_mode, norm, es);
  int G = GP > 0 ? 0 : pick_stage(a, cs_mode, norm, es, head_major);
  // Fewer tokens per block where their rows would take more than the LDS
  // budget: five or more resident blocks per compute unit keep enough bytes
  // in flight (a block holds its LDS from its first load to its last store).
  const int budget = env_int("MROPE_STAGE_G", 0) > 0 ? kStageLdsMax : kStageLdsTarget;
  auto fits = [&](int g) {
    // LDS, v's registers, and one thread per chunk position of a group
    return mrope::stage_lds_bytes(a.dtype, g, p) <= budget &&
           (int64_t)g * a.heads[2] * (a.D * es / 16) <= mrope::stage_max_v_chunks() &&
           g * (a.D * es / 16) <= mrope::kBlockThreads;
  };
  while (G > 1 && !fits(G)) G /= 2;
  if (G > 0 && !fits(G)) G = 0;
  if (GP > 0) {
    p.nt = GP;
    p.inv_cpr = 1.0f / (float)(a.D * es / 16);
    p.inv_run = 1.0f / (float)(GP * (a.D * es / 16));
    hrc = mrope::launch_planes(a.dtype, prec, p, tab, stream);
    g_last_kernel = "planes_kernel";
  } else if (G > 0) {
    p.stage_hm = head_major ? 1 : 0;
    p.inv_cpr = 1.0f / (float)(a.D * es / 16);
    for (int s = 0; s < kSlots; ++s) p.inv_heads[s] = 1.0f / (float)(a.heads[s] > 0 ? a.heads[s] : 1);
    p.waves_cap = waves_per_simd_stage();
    hrc = mrope::launch_stage(a.dtype, prec, G, p, tab, stream);
    g_last_kernel = "stage_kernel";
  } else if (use_flat(a, cs_mode, norm, v, es)) {
    p.inv_cpr = 1.0f / (float)(a.D / v);
    p.waves_cap = waves_per_simd_flat();
    hrc = mrope::launch_flat(a.dtype, v, prec, p, tab, stream);
    g_last_kernel = "flat_kernel";
  } else if (use_pipe(a, cs_mode, v, es)) {
    p.waves_cap = waves_per_simd(a, v, es);
    hrc = mrope::launch_qk_pipe(a.dtype, v, norm, prec, p, tab, stream);
    g_last_kernel = "qk_pipe_kernel";
  } else {
    p.waves_cap = waves_per_simd(a, v, es);
    hrc = mrope::launch_qk(a.dtype, v, cs_mode, norm, prec, p, tab, nt_cap, stream);
    g_last_kernel = "qk_kernel";
  }
  if (hrc != (int)hipSuccess)
    return fail(MROPE_EHIP, "kernel launch failed: %s", hipGetErrorString((hipError_t)hrc));
  return ok();
}

// Byte offsets of the regions of the position builder's workspace.
struct RopeWs {
  size_t sum = 0, carry = 0, valid = 0, end = 0, adv_i = 0, adv_v = 0, cum_t = 0, total = 0;
  int64_t chunks_per_sample = 0;
};

bool rope_ws_layout(int B, int64_t L, int n_img, int n_vid, RopeWs& w) {
  if (B < 0 || L < 0 || n_img < 0 || n_vid < 0) return false;
  w.chunks_per_sample = (L + mrope::kPosChunk - 1) / mrope::kPosChunk;
  const int64_t chunks = (int64_t)B * w.chunks_per_sample;
  // batch-wide filtered indices are packed as (index << 2 | type) in an int
  if ((int64_t)B * L >= (int64_t(1) << 29)) return false;
  (void)chunks;
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  size_t off = 0;
  w.sum = off;
  off = al(off + (size_t)chunks * mrope::kPosSumInts * 4);
  w.carry = off;
  off = al(off + (size_t)chunks * mrope::kPosCarryInts * 4);
  w.valid = off;
  off = al(off + (size_t)B * 4);
  w.end = off;
  off = al(off + (size_t)B * 12);
  w.adv_i = off;
  off = al(off + ((size_t)n_img + 1) * 8);
  w.adv_v = off;
  off = al(off + ((size_t)n_vid + 1) * 8);
  w.cum_t = off;
  off = al(off + ((size_t)n_vid + 1) * 4);
  w.total = off;
  return true;
}

Extent bytes_at(const void* base, int64_t n, int elem_bytes) {
  return extent_of(base, 1, 0, n, elem_bytes);
}

// Checks of the position builder's arguments other than the workspace.
int check_rope_index(const int32_t* mm_token_type, const int32_t* attention_mask, int batch,
                     int64_t seq_len, const int32_t* image_grid_thw, int n_images,
                     const int32_t* video_grid_thw, int n_videos, int spatial_merge,
                     int32_t* pos, int64_t pos_axis_stride, int32_t* rope_delta,
                     int32_t* status, RopeWs& w) {
  if (batch < 0 || seq_len < 0 || n_images < 0 || n_videos < 0)
    return fail(MROPE_EINVAL, "batch, seq_len, n_images and n_videos must be >= 0");
  if (spatial_merge < 1 || spatial_merge > 1024)
    return fail(MROPE_EINVAL, "spatial_merge = %d must be in [1, 1024]", spatial_merge);
  if (!rope_ws_layout(batch, seq_len, n_images, n_videos, w))
    return fail(MROPE_EUNSUPPORTED, "batch * seq_len is too large");
  const int64_t T = (int64_t)batch * seq_len;
  if (T > 0 && (mm_token_type == nullptr || pos == nullptr))
    return fail(MROPE_EINVAL, "mm_token_type and pos must be non-NULL");
  if (batch > 0 && rope_delta == nullptr) return fail(MROPE_EINVAL, "rope_delta is NULL");
  if (status == nullptr) return fail(MROPE_EINVAL, "status is NULL");
  if (n_images > 0 && image_grid_thw == nullptr) return fail(MROPE_EINVAL, "image_grid_thw is NULL");
  if (n_videos > 0 && video_grid_thw == nullptr) return fail(MROPE_EINVAL, "video_grid_thw is NULL");
  if (T > 0 && pos_axis_stride < T)
    return fail(MROPE_EINVAL, "pos_axis_stride %lld < batch*seq_len %lld",
                (long long)pos_axis_stride, (long long)T);
  for (const void* ptr : {(const void*)mm_token_type, (const void*)attention_mask,
                          (const void*)image_grid_thw, (const void*)video_grid_thw,
                          (const void*)pos, (const void*)rope_delta, (const void*)status})
    if (reinterpret_cast<uintptr_t>(ptr) % 4 != 0)
      return fail(MROPE_EINVAL, "int32 buffers must be 4-byte aligned");
  return MROPE_OK;
}

// Overlap checks of the outputs (and a caller workspace) against the inputs
// and one another.
int check_rope_index_overlaps(const int32_t* mm_token_type, const int32_t* attention_mask,
                              int batch, int64_t seq_len, const int32_t* image_grid_thw,
                              int n_images, const int32_t* video_grid_thw, int n_videos,
                              int32_t* pos, int64_t pos_axis_stride, int32_t* rope_delta,
                              int32_t* status, const void* workspace, size_t ws_bytes) {
  const int64_t T = (int64_t)batch * seq_len;
  const Extent outs[4] = {extent_of(pos, 3, pos_axis_stride, T, 4), bytes_at(rope_delta, batch, 4),
                          bytes_at(status, 1, 4), bytes_at(workspace, (int64_t)ws_bytes, 1)};
  const Extent ins[4] = {bytes_at(mm_token_type, T, 4), bytes_at(attention_mask, T, 4),
                         bytes_at(image_grid_thw, 3 * (int64_t)n_images, 4),
                         bytes_at(video_grid_thw, 3 * (int64_t)n_videos, 4)};
  for (int i = 0; i < 4; ++i) {
    for (int k = 0; k < 4; ++k)
      if (overlaps(outs[i], ins[k])) return fail(MROPE_EINVAL, "an output overlaps an input");
    for (int k = i + 1; k < 4; ++k)
      if (overlaps(outs[i], outs[k]))
        return fail(MROPE_EINVAL, "pos, rope_delta, status and workspace must not overlap");
  }
  return MROPE_OK;
}

// The launch of the three passes with a checked workspace.
int run_rope_index(const int32_t* mm_token_type, const int32_t* attention_mask, int batch,
                   int64_t seq_len, const int32_t* image_grid_thw, int n_images,
                   const int32_t* video_grid_thw, int n_videos, int spatial_merge, int32_t* pos,
                   int64_t pos_axis_stride, int32_t* rope_delta, int32_t* status,
                   void* workspace, const RopeWs& w, void* stream) {
  mrope::RopeIndexParams p;
  std::memset(&p, 0, sizeof(p));
  p.types = mm_token_type;
  p.mask = attention_mask;
  p.B = batch;
  p.L = seq_len;
  p.C = (int)w.chunks_per_sample;
  p.image_grid = image_grid_thw;
  p.n_images = n_images;
  p.video_grid = video_grid_thw;
  p.n_videos = n_videos;
  p.merge = spatial_merge;
  p.pos = pos;
  p.pos_stride = pos_axis_stride;
  p.rope_delta = rope_delta;
  p.status = status;
  char* ws = static_cast<char*>(workspace);
  p.ws_sum = reinterpret_cast<int32_t*>(ws + w.sum);
  p.ws_carry = reinterpret_cast<int32_t*>(ws + w.carry);
  p.ws_valid = reinterpret_cast<int32_t*>(ws + w.valid);
  p.ws_end = reinterpret_cast<int32_t*>(ws + w.end);
  p.ws_adv_i = reinterpret_cast<int64_t*>(ws + w.adv_i);
  p.ws_adv_v = reinterpret_cast<int64_t*>(ws + w.adv_v);
  p.ws_cum_t = reinterpret_cast<int32_t*>(ws + w.cum_t);
  const int hrc = mrope::launch_rope_index(p, stream, &g_last_kernel);
  if (hrc != (int)hipSuccess)
    return fail(MROPE_EHIP, "kernel launch failed: %s", hipGetErrorString((hipError_t)hrc));
  return ok();
}


}  // namespace

extern "C" {

int mrope_vision_qkv(const void* qkv, int64_t qkv_tok_stride, int64_t n, int heads, int D,
                     int rotary_dim, const int32_t* pos, int64_t pos_axis_stride, double theta,
                     int dtype, int precision, void* q_out, void* k_out, void* v_out,
                     int64_t out_head_stride, int64_t out_tok_stride, const float* cs_cache,
                     int cache_rows, void* stream) {
  if (heads < 0) return fail(MROPE_EINVAL, "heads = %d is negative", heads);
  QKArgs a;
  std::memset(&a, 0, sizeof(a));
  const int es = elem_bytes_of(dtype);
  const int64_t plane = (int64_t)heads * D;
  if (qkv_tok_stride < 3 * plane)
    return fail(MROPE_EINVAL, "qkv token stride %lld < 3*heads*D = %lld",
                (long long)qkv_tok_stride, (long long)(3 * plane));
  void* outs[3] = {q_out, k_out, v_out};
  for (int s = 0; s < 3; ++s) {
    a.x[s] = qkv == nullptr ? nullptr : static_cast<const char*>(qkv) + s * plane * es;
    a.x_ts[s] = qkv_tok_stride;
    a.heads[s] = (s == 2 && v_out == nullptr) ? 0 : heads;
    a.y[s] = outs[s];
    a.y_ts[s] = out_tok_stride;
    a.y_hs[s] = out_head_stride;
  }
  if (n > 0 && (out_head_stride <= 0 || out_tok_stride <= 0))
    return fail(MROPE_EINVAL, "output strides must be positive");
  a.T = n;
  a.D = D;
  a.rd = rotary_dim;
  a.dtype = dtype;
  a.precision = precision;
  int rc = check_qk_tensors(a, true);
  if (rc) return rc;
  if (!(theta > 0.0) || !std::isfinite(theta))
    return fail(MROPE_EINVAL, "theta must be positive and finite");
  mrope::ColTable tab;
  std::memset(&tab, 0, sizeof(tab));
  rc = build_table(rotary_dim, theta, nullptr, 0, MROPE_LAYOUT_VISION_2D, nullptr, tab);
  if (rc) return rc;
  if (pos_axis_stride < 0) return fail(MROPE_EINVAL, "pos_axis_stride is negative");
  if (n > 0 && heads > 0 && pos == nullptr) return fail(MROPE_EINVAL, "pos is NULL");
  CacheArgs ca;
  Extent cache_ext;
  rc = check_cache(cs_cache, cache_rows, rotary_dim / 4, ca, cache_ext);
  if (rc) return rc;
  Extent extra[2] = {extent_of(pos, 2, pos_axis_stride, n, 4), cache_ext};
  return run_qk(a, mrope::kCsFromPositions, false, tab, pos, pos_axis_stride, nullptr, nullptr, 0,
                0.0f, stream, extra, 2, nullptr, &ca);
}

int mrope_cos_sin_cache(int dim, double theta, int rows, float* cache, void* stream) {
  if (dim <= 0 || dim % 2 != 0 || dim > MROPE_MAX_ROTARY_DIM)
    return fail(MROPE_EINVAL, "dim = %d must be even and in (0, %d]", dim, MROPE_MAX_ROTARY_DIM);
  if (!(theta > 0.0) || !std::isfinite(theta))
    return fail(MROPE_EINVAL, "theta must be positive and finite");
  if (rows < 0) return fail(MROPE_EINVAL, "rows is negative");
  if (rows > 0 && cache == nullptr) return fail(MROPE_EINVAL, "cache is NULL");
  if (reinterpret_cast<uintptr_t>(cache) % 8 != 0)
    return fail(MROPE_EINVAL, "cache must be 8-byte aligned");
  if (rows == 0) return ok();
  mrope::ColTable tab;
  std::memset(&tab, 0, sizeof(tab));
  fill_inv(dim, theta, tab.inv);
  const int hrc = mrope::launch_cos_sin_cache(tab, dim / 2, rows, cache, stream);
  if (hrc != (int)hipSuccess)
    return fail(MROPE_EHIP, "kernel launch failed: %s", hipGetErrorString((hipError_t)hrc));
  return ok();
}

size_t mrope_rope_index_workspace_size(int batch, int64_t seq_len, int n_images, int n_videos) {
  RopeWs w;
  if (!rope_ws_layout(batch, seq_len, n_images, n_videos, w)) return 0;
  return w.total;
}

int mrope_rope_index(const int32_t* mm_token_type, const int32_t* attention_mask, int batch,
                     int64_t seq_len, const int32_t* image_grid_thw, int n_images,
                     const int32_t* video_grid_thw, int n_videos, int spatial_merge,
                     int32_t* pos, int64_t pos_axis_stride, int32_t* rope_delta,
                     int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  RopeWs w;
  int rc = check_rope_index(mm_token_type, attention_mask, batch, seq_len, image_grid_thw,
                            n_images, video_grid_thw, n_videos, spatial_merge, pos,
                            pos_axis_stride, rope_delta, status, w);
  if (rc) return rc;
  if (workspace == nullptr || workspace_bytes < w.total)
    return fail(MROPE_EINVAL, "workspace of %zu bytes needed (got %zu)", w.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 8 != 0)
    return fail(MROPE_EINVAL, "workspace must be 8-byte aligned");
  rc = check_rope_index_overlaps(mm_token_type, attention_mask, batch, seq_len, image_grid_thw,
                                 n_images, video_grid_thw, n_videos, pos, pos_axis_stride,
                                 rope_delta, status, workspace, w.total);
  if (rc) return rc;
  return run_rope_index(mm_token_type, attention_mask, batch, seq_len, image_grid_thw, n_images,
                        video_grid_thw, n_videos, spatial_merge, pos, pos_axis_stride,
                        rope_delta, status, workspace, w, stream);
}

int mrope_rope_index_noalloc(const int32_t* mm_token_type, const int32_t* attention_mask,
                             int batch, int64_t seq_len, const int32_t* image_grid_thw,
                             int n_images, const int32_t* video_grid_thw, int n_videos,
                             int spatial_merge, int32_t* pos, int64_t pos_axis_stride,
                             int32_t* rope_delta, int32_t* status, void* stream) {
  RopeWs w;
  int rc = check_rope_index(mm_token_type, attention_mask, batch, seq_len, image_grid_thw,
                            n_images, video_grid_thw, n_videos, spatial_merge, pos,
                            pos_axis_stride, rope_delta, status, w);
  if (rc) return rc;
  if (w.total > mrope::kRopeIndexScratchBytes)
    return fail(MROPE_EUNSUPPORTED,
                "these sizes need %zu bytes of workspace; the static workspace of "
                "mrope_rope_index_noalloc holds %zu (use mrope_rope_index with a workspace)",
                w.total, mrope::kRopeIndexScratchBytes);
  rc = check_rope_index_overlaps(mm_token_type, attention_mask, batch, seq_len, image_grid_thw,
                                 n_images, video_grid_thw, n_videos, pos, pos_axis_stride,
                                 rope_delta, status, nullptr, 0);
  if (rc) return rc;
  void* scratch = nullptr;
  const int hrc = mrope::rope_index_scratch(&scratch);
  if (hrc != (int)hipSuccess)
    return fail(MROPE_EHIP, "the static workspace's device address: %s",
                hipGetErrorString((hipError_t)hrc));
  return run_rope_index(mm_token_type, attention_mask, batch, seq_len, image_grid_thw, n_images,
                        video_grid_thw, n_videos, spatial_merge, pos, pos_axis_stride,
                        rope_delta, status, scratch, w, stream);
}

int mrope_vision_pos_ids(const int32_t* grid_thw, int n_images, int spatial_merge,
                         int64_t n_tokens, int32_t* pos, int64_t pos_axis_stride,
                         int32_t* status, void* stream) {
  if (n_images < 0 || n_images > mrope::kMaxVisionImages)
    return fail(MROPE_EINVAL, "n_images = %d must be in [0, %d]", n_images,
                mrope::kMaxVisionImages);
  if (spatial_merge < 1 || spatial_merge > 1024)
    return fail(MROPE_EINVAL, "spatial_merge = %d must be in [1, 1024]", spatial_merge);
  if (n_tokens < 0) return fail(MROPE_EINVAL, "n_tokens is negative");
  if (n_images > 0 && grid_thw == nullptr) return fail(MROPE_EINVAL, "grid_thw is NULL");
  if (n_tokens > 0 && pos == nullptr) return fail(MROPE_EINVAL, "pos is NULL");
  if (status == nullptr) return fail(MROPE_EINVAL, "status is NULL");
  if (n_tokens > 0 && pos_axis_stride < n_tokens)
    return fail(MROPE_EINVAL, "pos_axis_stride < n_tokens");
  for (const void* ptr : {(const void*)grid_thw, (const void*)pos, (const void*)status})
    if (reinterpret_cast<uintptr_t>(ptr) % 4 != 0)
      return fail(MROPE_EINVAL, "int32 buffers must be 4-byte aligned");
  const Extent pe = extent_of(pos, 2, pos_axis_stride, n_tokens, 4);
  const Extent ge = bytes_at(grid_thw, 3 * (int64_t)n_images, 4);
  const Extent se = bytes_at(status, 1, 4);
  if (overlaps(pe, ge) || overlaps(pe, se) || overlaps(se, ge))
    return fail(MROPE_EINVAL, "pos, status and grid_thw must not overlap");
  mrope::VisionPosParams p;
  std::memset(&p, 0, sizeof(p));
  p.grid = grid_thw;
  p.n_images = n_images;
  p.merge = spatial_merge;
  p.N = n_tokens;
  p.pos = pos;
  p.pos_stride = pos_axis_stride;
  p.status = status;
  const int hrc = mrope::launch_vision_pos_ids(p, stream);
  if (hrc != (int)hipSuccess)
    return fail(MROPE_EHIP, "kernel launch failed: %s", hipGetErrorString((hipError_t)hrc));
  return ok();
}

int mrope_inv_freq(int dim, double theta, float* out) {
  if (out == nullptr) return fail(MROPE_EINVAL, "out is NULL");
  if (dim <= 0 || dim % 2 != 0) return fail(MROPE_EINVAL, "dim = %d must be positive and even", dim);
  if (!(theta > 0.0) || !std::isfinite(theta))
    return fail(MROPE_EINVAL, "theta must be positive and finite");
  fill_inv(dim, theta, out);
  return ok();
}

int mrope_axis_table(int half, const int* section, int n_sections, int layout,
                     uint8_t* axis_out) {
  if (axis_out == nullptr) return fail(MROPE_EINVAL, "axis_out is NULL");
  const int rc = build_axis(half, section, n_sections, layout, axis_out);
  return rc ? rc : ok();
}

int mrope_cos_sin(const int32_t* pos, int64_t pos_axis_stride, int n_axes, int64_t T,
                  const float* inv_freq, const int* section, int n_sections, int layout,
                  int rotary_dim, float* cos_out, float* sin_out, int64_t cs_tok_stride,
                  void* stream) {
  if (T < 0) return fail(MROPE_EINVAL, "T is negative");
  if (rotary_dim <= 0 || rotary_dim % 2 != 0)
    return fail(MROPE_EINVAL, "rotary_dim = %d must be positive and even", rotary_dim);
  if (rotary_dim > MROPE_MAX_ROTARY_DIM)
    return fail(MROPE_EUNSUPPORTED, "rotary_dim = %d exceeds %d", rotary_dim, MROPE_MAX_ROTARY_DIM);
  if (inv_freq == nullptr) return fail(MROPE_EINVAL, "inv_freq is NULL");
  mrope::ColTable tab;
  int rc = build_table(rotary_dim, 0.0, section, n_sections, layout, inv_freq, tab);
  if (rc) return rc;
  if (n_axes != expected_axes(layout, n_sections))
    return fail(MROPE_EINVAL, "n_axes = %d does not match the layout (%d)", n_axes,
                expected_axes(layout, n_sections));
  if (pos_axis_stride < 0) return fail(MROPE_EINVAL, "pos_axis_stride is negative");
  if (cs_tok_stride < rotary_dim)
    return fail(MROPE_EINVAL, "cs_tok_stride %lld < rotary_dim %d", (long long)cs_tok_stride,
                rotary_dim);
  if (T == 0) return ok();
  if (pos == nullptr || cos_out == nullptr || sin_out == nullptr)
    return fail(MROPE_EINVAL, "pos, cos_out and sin_out must be non-NULL");
  const Extent ce = extent_of(cos_out, T, cs_tok_stride, rotary_dim, 4);
  const Extent se = extent_of(sin_out, T, cs_tok_stride, rotary_dim, 4);
  const Extent pe = extent_of(pos, n_axes, pos_axis_stride, T, 4);
  if (overlaps(ce, se) || overlaps(ce, pe) || overlaps(se, pe))
    return fail(MROPE_EINVAL, "cos_out, sin_out and pos must not overlap");
  mrope::CosSinParams p;
  p.pos = pos;
  p.pos_stride = pos_axis_stride;
  p.T = T;
  p.half = rotary_dim / 2;
  p.rd = rotary_dim;
  p.cos = cos_out;
  p.sin = sin_out;
  p.cs_ts = cs_tok_stride;
  const int hrc = mrope::launch_cos_sin(p, tab, stream);
  if (hrc != (int)hipSuccess)
    return fail(MROPE_EHIP, "kernel launch failed: %s", hipGetErrorString((hipError_t)hrc));
  return ok();
}

int rms_norm(const void* x, int64_t x_tok_stride, int64_t T, int heads, int D, const void* w,
             float eps, int dtype, void* out, int64_t out_tok_stride, void* stream) {
  QKArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x[0] = x;
  a.x_ts[0] = x_tok_stride;
  a.heads[0] = heads;
  a.y[0] = out;
  a.y_ts[0] = out_tok_stride;
  a.w[0] = w;
  a.T = T;
  a.D = D;
  a.rd = 0;
  a.dtype = dtype;
  int rc = check_qk_tensors(a, false);
  if (rc) return rc;
  if (!std::isfinite(eps) || eps < 0.0f) return fail(MROPE_EINVAL, "eps must be finite and >= 0");
  if (T > 0 && heads > 0 && w == nullptr) return fail(MROPE_EINVAL, "w is NULL");
  mrope::ColTable tab;
  std::memset(&tab, 0, sizeof(tab));
  return run_qk(a, mrope::kCsNone, true, tab, nullptr, 0, nullptr, nullptr, 0, eps, stream,
                nullptr, 0);
}

int apply_rotary_qk(const void* q, int64_t q_tok_stride, int hq, const void* k,
                    int64_t k_tok_stride, int hk, int64_t T, int D, int rotary_dim,
                    const float* cos, const float* sin, int64_t cs_tok_stride, int dtype,
                    int precision, void* q_out, int64_t q_out_tok_stride, void* k_out,
                    int64_t k_out_tok_stride, void* stream) {
  QKArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x[0] = q;
  a.x[1] = k;
  a.x_ts[0] = q_tok_stride;
  a.x_ts[1] = k_tok_stride;
  a.heads[0] = hq;
  a.heads[1] = hk;
  a.y[0] = q_out;
  a.y[1] = k_out;
  a.y_ts[0] = q_out_tok_stride;
  a.y_ts[1] = k_out_tok_stride;
  a.T = T;
  a.D = D;
  a.rd = rotary_dim;
  a.dtype = dtype;
  a.precision = precision;
  int rc = check_qk_tensors(a, true);
  if (rc) return rc;
  if (cs_tok_stride < rotary_dim)
    return fail(MROPE_EINVAL, "cs_tok_stride %lld < rotary_dim %d", (long long)cs_tok_stride,
                rotary_dim);
  if (T > 0 && hq + hk > 0 && (cos == nullptr || sin == nullptr))
    return fail(MROPE_EINVAL, "cos and sin must be non-NULL");
  Extent extra[2] = {extent_of(cos, T, cs_tok_stride, rotary_dim, 4),
                     extent_of(sin, T, cs_tok_stride, rotary_dim, 4)};
  mrope::ColTable tab;
  std::memset(&tab, 0, sizeof(tab));
  return run_qk(a, mrope::kCsFromTable, false, tab, nullptr, 0, cos, sin, cs_tok_stride, 0.0f,
                stream, extra, 2);
}

int rmsnorm_mrope_qk(const void* q, int64_t q_tok_stride, int hq, const void* k,
                     int64_t k_tok_stride, int hk, int64_t T, int D, int rotary_dim,
                     const int32_t* pos, int64_t pos_axis_stride, int n_axes,
                     const int* section, int n_sections, int layout, double theta,
                     const void* wq, const void* wk, float eps, int dtype, int precision,
                     void* q_out, int64_t q_out_tok_stride, void* k_out,
                     int64_t k_out_tok_stride, void* stream) {
  return rmsnorm_mrope_qk_cached(q, q_tok_stride, hq, k, k_tok_stride, hk, T, D, rotary_dim, pos,
                                 pos_axis_stride, n_axes, section, n_sections, layout, theta, wq,
                                 wk, eps, dtype, precision, q_out, q_out_tok_stride, k_out,
                                 k_out_tok_stride, nullptr, 0, stream);
}

int rmsnorm_mrope_qk_cached(const void* q, int64_t q_tok_stride, int hq, const void* k,
                            int64_t k_tok_stride, int hk, int64_t T, int D, int rotary_dim,
                            const int32_t* pos, int64_t pos_axis_stride, int n_axes,
                            const int* section, int n_sections, int layout, double theta,
                            const void* wq, const void* wk, float eps, int dtype, int precision,
                            void* q_out, int64_t q_out_tok_stride, void* k_out,
                            int64_t k_out_tok_stride, const float* cs_cache, int cache_rows,
                            void* stream) {
  QKArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x[0] = q;
  a.x[1] = k;
  a.x_ts[0] = q_tok_stride;
  a.x_ts[1] = k_tok_stride;
  a.heads[0] = hq;
  a.heads[1] = hk;
  a.y[0] = q_out;
  a.y[1] = k_out;
  a.y_ts[0] = q_out_tok_stride;
  a.y_ts[1] = k_out_tok_stride;
  a.w[0] = wq;
  a.w[1] = wk;
  a.T = T;
  a.D = D;
  a.rd = rotary_dim;
  a.dtype = dtype;
  a.precision = precision;
  int rc = check_qk_tensors(a, true);
  if (rc) return rc;
  if ((wq == nullptr) != (wk == nullptr))
    return fail(MROPE_EINVAL, "wq and wk must both be given or both be NULL");
  const bool norm = wq != nullptr;
  if (norm && (!std::isfinite(eps) || eps < 0.0f))
    return fail(MROPE_EINVAL, "eps must be finite and >= 0");
  if (!(theta > 0.0) || !std::isfinite(theta))
    return fail(MROPE_EINVAL, "theta must be positive and finite");
  mrope::ColTable tab;
  std::memset(&tab, 0, sizeof(tab));
  rc = build_table(rotary_dim, theta, section, n_sections, layout, nullptr, tab);
  if (rc) return rc;
  if (n_axes != expected_axes(layout, n_sections))
    return fail(MROPE_EINVAL, "n_axes = %d does not match the layout (%d)", n_axes,
                expected_axes(layout, n_sections));
  if (pos_axis_stride < 0) return fail(MROPE_EINVAL, "pos_axis_stride is negative");
  if (T > 0 && hq + hk > 0 && pos == nullptr) return fail(MROPE_EINVAL, "pos is NULL");
  const int half = rotary_dim / 2;
  CacheArgs ca;
  Extent cache_ext;
  rc = check_cache(cs_cache, cache_rows, layout == MROPE_LAYOUT_VISION_2D ? half / 2 : half, ca,
                   cache_ext);
  if (rc) return rc;
  Extent extra[2] = {extent_of(pos, n_axes, pos_axis_stride, T, 4), cache_ext};
  return run_qk(a, mrope::kCsFromPositions, norm, tab, pos, pos_axis_stride, nullptr, nullptr, 0,
                eps, stream, extra, 2, nullptr, &ca);
}

int mrope_decode_qk(const void* q, int64_t q_tok_stride, int hq, const void* k,
                    int64_t k_tok_stride, int hk, int batch, int new_tokens, int D,
                    int rotary_dim, const int32_t* cache_len, const int32_t* rope_delta,
                    double theta, const void* wq, const void* wk, float eps, int dtype,
                    int precision, void* q_out, int64_t q_out_tok_stride, void* k_cache,
                    int64_t k_cache_seq_stride, int64_t k_cache_tok_stride, int k_cache_capacity,
                    void* stream) {
  if (batch < 0 || new_tokens < 0)
    return fail(MROPE_EINVAL, "batch = %d and new_tokens = %d must be >= 0", batch, new_tokens);
  const int64_t T = (int64_t)batch * new_tokens;
  QKArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x[0] = q;
  a.x[1] = k;
  a.x_ts[0] = q_tok_stride;
  a.x_ts[1] = k_tok_stride;
  a.heads[0] = hq;
  a.heads[1] = hk;
  a.y[0] = q_out;
  a.y[1] = k_cache;
  a.y_ts[0] = q_out_tok_stride;
  a.y_ts[1] = (int64_t)hk * D;  // one row at a time; the cache layout is checked below
  a.w[0] = wq;
  a.w[1] = wk;
  a.T = T;
  a.D = D;
  a.rd = rotary_dim;
  a.dtype = dtype;
  a.precision = precision;
  int rc = check_qk_tensors(a, true);
  if (rc) return rc;
  if ((wq == nullptr) != (wk == nullptr))
    return fail(MROPE_EINVAL, "wq and wk must both be given or both be NULL");
  const bool norm = wq != nullptr;
  if (norm && (!std::isfinite(eps) || eps < 0.0f))
    return fail(MROPE_EINVAL, "eps must be finite and >= 0");
  if (!(theta > 0.0) || !std::isfinite(theta))
    return fail(MROPE_EINVAL, "theta must be positive and finite");
  if (T > 0 && cache_len == nullptr) return fail(MROPE_EINVAL, "cache_len is NULL");
  const int es = elem_bytes_of(dtype);
  Extent cache_ext;
  if (T > 0 && hk > 0) {
    if (k_cache_capacity < 1) return fail(MROPE_EINVAL, "k_cache_capacity must be >= 1");
    if (k_cache_tok_stride < (int64_t)hk * D)
      return fail(MROPE_EINVAL, "k_cache_tok_stride %lld < hk*D", (long long)k_cache_tok_stride);
    if (batch > 1 && k_cache_seq_stride < (int64_t)k_cache_capacity * k_cache_tok_stride)
      return fail(MROPE_EINVAL, "k_cache_seq_stride is smaller than capacity * tok_stride");
    cache_ext = extent_of(k_cache, 1,
                          0, ((int64_t)(batch - 1) * k_cache_seq_stride +
                              (int64_t)(k_cache_capacity - 1) * k_cache_tok_stride +
                              (int64_t)hk * D), es);
    const Extent qin = extent_of(q, T, q_tok_stride, (int64_t)hq * D, es);
    const Extent kin = extent_of(k, T, k_tok_stride, (int64_t)hk * D, es);
    const Extent qout = extent_of(q_out, T, q_out_tok_stride, (int64_t)hq * D, es);
    if (overlaps(cache_ext, qin) || overlaps(cache_ext, kin) || overlaps(cache_ext, qout))
      return fail(MROPE_EINVAL, "k_cache overlaps q, k or q_out");
    if (norm && (overlaps(cache_ext, extent_of(wq, 1, D, D, es)) ||
                 overlaps(cache_ext, extent_of(wk, 1, D, D, es))))
      return fail(MROPE_EINVAL, "k_cache overlaps a weight vector");
  }
  mrope::ColTable tab;
  std::memset(&tab, 0, sizeof(tab));
  // Text positions: every column reads the same position, so one chunked
  // section covering all columns is the 1-D RoPE table.
  const int half = rotary_dim / 2;
  rc = build_table(rotary_dim, theta, &half, 1, MROPE_LAYOUT_CHUNKED, nullptr, tab);
  if (rc) return rc;
  Extent extra[2] = {extent_of(cache_len, 1, 0, batch, 4),
                     extent_of(rope_delta, 1, 0, batch, 4)};
  DecodeArgs dec;
  dec.cache_len = cache_len;
  dec.rope_delta = rope_delta;
  dec.new_tokens = new_tokens;
  dec.kc_seq = k_cache_seq_stride;
  dec.kc_tok = k_cache_tok_stride;
  dec.kc_cap = k_cache_capacity;
  if (hk > 0 && T > 0)
    for (const Extent& e : extra)
      if (overlaps(cache_ext, e)) return fail(MROPE_EINVAL, "k_cache overlaps cache_len/rope_delta");
  return run_qk(a, mrope::kCsDecode, norm, tab, nullptr, 0, nullptr, nullptr, 0, eps, stream,
                extra, 2, &dec);
}

int mrope_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0) return fail(MROPE_EINVAL, "bytes = %lld is negative", (long long)bytes);
  if (bytes % 16 != 0) return fail(MROPE_EINVAL, "bytes = %lld is not a multiple of 16",
                                   (long long)bytes);
  if (bytes > (int64_t(1) << 40))
    return fail(MROPE_EUNSUPPORTED, "bytes = %lld exceeds 2^40", (long long)bytes);
  if (bytes == 0) return ok();
  if (src == nullptr || dst == nullptr) return fail(MROPE_EINVAL, "src and dst must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
    return fail(MROPE_EINVAL, "src and dst must be 16-byte aligned");
  if (overlaps(bytes_at(src, bytes, 1), bytes_at(dst, bytes, 1)))
    return fail(MROPE_EINVAL, "src and dst overlap");
  const int hrc = mrope::launch_stream_copy(src, dst, bytes, stream);
  if (hrc != (int)hipSuccess)
    return fail(MROPE_EHIP, "kernel launch failed: %s", hipGetErrorString((hipError_t)hrc));
  return ok();
}

const char* mrope_last_error(void) { return g_err.c_str(); }

const char* mrope_last_kernel(void) { return g_last_kernel; }

}  // extern "C"
