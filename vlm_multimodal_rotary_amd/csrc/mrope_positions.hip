// Position builders for multimodal rotary embedding on gfx950.
//
// rope_index: the 3-axis (T, H, W) position table of a batch of mixed text /
// image / video token sequences plus the per-sample rope_deltas ("Interleaved
// Rotary Position Embedding", get_rope_index walkthrough).  Every position is
// a prefix quantity of the token sequence, so the builder is three scans:
//
//   1. summarize: one block per 1024-token chunk of a sample reduces the
//      chunk (valid and text token counts, first/last valid type, segment
//      starts by type, the last start) -- tokens are read once.
//   2. carry:     one block scans the chunk summaries (held in LDS when they
//      fit) and writes each chunk's carry-in: filtered index, text count, the
//      previous valid type, the global image / video grid counters, the open
//      segment; it also builds the grid-advance prefix tables and the
//      per-sample valid length.
//   3. apply:     one block per chunk re-reads its tokens, resolves segment
//      starts with block scans seeded by the carry, and writes the positions;
//      rope_delta = max + 1 - valid length by one atomic max per block.
//
// When the chunk summaries fit LDS (up to 1024 chunks) and the grids fit the
// LDS tables, passes 2 and 3 run as one kernel: every block of the apply pass
// does the carry work itself, in LDS, and keeps its own chunk's carry.
//
// The grid iterators of the walkthrough (one image iterator and one video
// iterator shared by the batch, videos split into single-slice grids) become
// global counters: the k-th image segment of the batch uses image grid k, the
// k-th video segment uses slice k of the concatenated video slices.
//
// vision_pos_ids: (row, col) of every vision patch in merge-block order,
// repeated per frame ("Qwen3-VL" walkthrough, rot_pos_emb): one thread per
// patch, the image found by binary search over the grids' patch counts.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "mrope_internal.h"

// Workspace of mrope_rope_index_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  In host code this name is a
// host-side stand-in, not a device address: only the address that
// hipGetSymbolAddress returns on each device reaches a kernel.
static __device__ __align__(256) unsigned char scratch[mrope::kRopeIndexScratchBytes];

namespace mrope {

int rope_index_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t rc = hipGetDevice(&dev);
  if (rc != hipSuccess) return (int)rc;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    rc = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (rc != hipSuccess) return (int)rc;
    ptrs[dev] = ptr;
  }
  *out = ptrs[dev];
  return (int)hipSuccess;
}

namespace {

constexpr int kPT = kPosThreads;

// Raw buffer over `bytes` bytes at base: loads past the range return 0 and
// touch no memory, so a lane with nothing to read needs no branch.
__device__ __forceinline__ int32_t load_in_range(const int32_t* base, uint32_t count, int i) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(base), 0, (int)(count * sizeof(int32_t)), 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)i * (uint32_t)sizeof(int32_t), 0, 0);
}
constexpr int kPer = kPosPerThread;
constexpr int kWaves = kPT / kWaveSize;

// ---------------------------------------------------------------------------
// Block scans over 256 threads (four wavefronts).
// ---------------------------------------------------------------------------

// Wavefront scans on DPP moves (register-to-register, no LDS round trip).
// A lane whose DPP source lies outside its row, or whose row the row mask
// leaves out, receives `id` instead.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_move(int id, int v) {
  return __builtin_amdgcn_update_dpp(id, v, CTRL, ROW_MASK, 0xF, false);
}

template <int CTRL, int ROW_MASK, typename T>
__device__ __forceinline__ T dpp_move(T id, T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit lanes");
  if constexpr (sizeof(T) == 4) {
    return (T)dpp_move<CTRL, ROW_MASK>((int)id, (int)v);
  } else {
    const unsigned long long u = (unsigned long long)v, d = (unsigned long long)id;
    const unsigned lo = (unsigned)dpp_move<CTRL, ROW_MASK>((int)(unsigned)d, (int)(unsigned)u);
    const unsigned hi =
        (unsigned)dpp_move<CTRL, ROW_MASK>((int)(unsigned)(d >> 32), (int)(unsigned)(u >> 32));
    return (T)(((unsigned long long)hi << 32) | lo);
  }
}

// Inclusive scan over the wavefront: Hillis-Steele within each row of 16
// lanes (row_shr 1, 2, 4, 8), then the last lane of row 0 and 2 into rows 1
// and 3 (row_bcast 15) and the last lane of row 1 into rows 2 and 3
// (row_bcast 31).
template <typename T, typename Op>
__device__ __forceinline__ T wave_incl_scan(T v, T id, Op op) {
  v = op(v, dpp_move<0x111, 0xF>(id, v));
  v = op(v, dpp_move<0x112, 0xF>(id, v));
  v = op(v, dpp_move<0x114, 0xF>(id, v));
  v = op(v, dpp_move<0x118, 0xF>(id, v));
  v = op(v, dpp_move<0x142, 0xA>(id, v));
  v = op(v, dpp_move<0x143, 0xC>(id, v));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_incl_sum(T v) {
  return wave_incl_scan(v, (T)0, [](T a, T b) { return a + b; });
}

template <typename T>
__device__ __forceinline__ T wave_incl_max(T v, T lo) {
  return wave_incl_scan(v, lo, [](T a, T b) { return a > b ? a : b; });
}

// Exclusive sum over the block; *total receives the block sum.  `sh` holds
// kWaves entries.  Contains barriers: every thread of the block calls it.
template <typename T>
__device__ T block_excl_sum(T v, T* total, T* sh) {
  const int w = threadIdx.x / kWaveSize;
  const int lane = threadIdx.x & (kWaveSize - 1);
  const T incl = wave_incl_sum(v);
  if (lane == kWaveSize - 1) sh[w] = incl;
  __syncthreads();
  T before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const T s = sh[i];
    if (i < w) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Exclusive max over the block (identity `lo`); *total receives the block max.
template <typename T>
__device__ T block_excl_max(T v, T lo, T* total, T* sh) {
  const int w = threadIdx.x / kWaveSize;
  const int lane = threadIdx.x & (kWaveSize - 1);
  const T incl = wave_incl_max(v, lo);
  const T prev = dpp_move<0x138, 0xF>(lo, incl);   // wave_shr 1: the lane before
  if (lane == kWaveSize - 1) sh[w] = incl;
  __syncthreads();
  T before = lo, all = lo;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const T s = sh[i];
    if (i < w && s > before) before = s;
    if (s > all) all = s;
  }
  __syncthreads();
  *total = all;
  return prev > before ? prev : before;
}

// Several independent exclusive scans in one LDS round (two barriers in all).
// kind[k]: 0 sum, 1 max, 2 bitwise or; id[k] is the identity of the k-th
// scan; excl[k] receives the scan before this thread, total[k] the block's.
// `sh` holds K * kWaves entries.  Contains barriers: every thread calls it.
enum ScanKind : int { kScanSum = 0, kScanMax = 1, kScanOr = 2 };

template <typename T>
__device__ __forceinline__ T scan_op(int kind, T a, T b) {
  return kind == kScanSum ? a + b : kind == kScanMax ? (a > b ? a : b) : (a | b);
}

template <int K, typename T>
__device__ __forceinline__ void block_scan_multi(const T (&v)[K], const T (&id)[K],
                                                 const int (&kind)[K], T (&excl)[K],
                                                 T (&total)[K], T* sh) {
  const int w = threadIdx.x / kWaveSize;
  const int lane = threadIdx.x & (kWaveSize - 1);
  T prev[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int kd = kind[k];
    const T incl = wave_incl_scan(v[k], id[k], [kd](T a, T b) { return scan_op(kd, a, b); });
    prev[k] = dpp_move<0x138, 0xF>(id[k], incl);   // wave_shr 1: the lane before
    if (lane == kWaveSize - 1) sh[k * kWaves + w] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    T before = id[k], all = id[k];
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const T x = sh[k * kWaves + i];
      if (i < w) before = scan_op(kind[k], before, x);
      all = scan_op(kind[k], all, x);
    }
    excl[k] = scan_op(kind[k], before, prev[k]);
    total[k] = all;
  }
  __syncthreads();
}

// Bitwise OR over the block.
__device__ int block_or(int v, int* sh) {
  const int w = threadIdx.x / kWaveSize;
  const int lane = threadIdx.x & (kWaveSize - 1);
  v = wave_incl_scan(v, 0, [](int a, int b) { return a | b; });
  if (lane == kWaveSize - 1) sh[w] = v;
  __syncthreads();
  int all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) all |= sh[i];
  __syncthreads();
  return all;
}

// ---------------------------------------------------------------------------
// Per-thread walk over its run of kPer tokens (shared by summarize / apply).
// ---------------------------------------------------------------------------

struct Run {
  int ty[kPer];      // token type (bad values mapped to text), -1 = not valid
  int nv, nt;        // valid tokens, valid text tokens
  int ft, lt;        // first / last valid type of the run, -1 if none
  int ni, nvd;       // starts after the run's first valid token, by type
  int lsF, lsT;      // run-local filtered index and type of the last such start
  int flags;
};

// The run's token types and mask words.  Loads at clamped addresses, issued
// together; tokens past the row are discarded by parse_run.  Without a mask
// the type row is read in its place, so no branch surrounds a load.
struct RunWords {
  int tv[kPer], mv[kPer];
};

__device__ __forceinline__ void load_run(const RopeIndexParams& p, int b, int64_t l0,
                                         RunWords& w) {
  const int64_t row = (int64_t)b * p.L;
  const int32_t* mrow = p.mask != nullptr ? p.mask : p.types;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t l = (l0 + k) < p.L ? (l0 + k) : (p.L - 1);
    w.tv[k] = p.types[row + l];
    w.mv[k] = mrow[row + l];
  }
}

__device__ __forceinline__ void parse_run(const RopeIndexParams& p, int64_t l0,
                                          const RunWords& w, Run& r) {
  r.nv = r.nt = r.ni = r.nvd = 0;
  r.ft = r.lt = r.lsF = r.lsT = -1;
  r.flags = 0;
  const bool masked = p.mask != nullptr;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    int ty = -1;
    if (l0 + k < p.L && (!masked || w.mv[k] != 0)) {
      ty = w.tv[k];
      if (ty < 0 || ty > 2) {
        r.flags |= MROPE_POS_BAD_TYPE;
        ty = 0;
      }
    }
    r.ty[k] = ty;
    if (ty < 0) continue;
    if (r.ft < 0) {
      r.ft = ty;
    } else if (ty != r.lt) {
      r.ni += ty == 1;
      r.nvd += ty == 2;
      r.lsF = r.nv;
      r.lsT = ty;
    }
    r.lt = ty;
    ++r.nv;
    r.nt += ty == 0;
  }
}

__device__ __forceinline__ void read_run(const RopeIndexParams& p, int b, int64_t l0, Run& r) {
  RunWords w;
  load_run(p, b, l0, w);
  parse_run(p, l0, w, r);
}

// ---------------------------------------------------------------------------
// Pass 1: chunk summaries.
// ---------------------------------------------------------------------------

// Four per-run counts packed in 16-bit fields of one 64-bit word (a block
// holds at most kPosChunk = 1024 tokens, so no field carries into the next).
__device__ __forceinline__ unsigned long long pack4(int a, int b, int c, int d) {
  return (unsigned long long)a | ((unsigned long long)b << 16) | ((unsigned long long)c << 32) |
         ((unsigned long long)d << 48);
}

__device__ __forceinline__ int field(unsigned long long v, int i) {
  return (int)((v >> (16 * i)) & 0xFFFFu);
}

__global__ void __launch_bounds__(kPT) rope_index_summarize(const RopeIndexParams p) {
  __shared__ int sh[kWaves];
  __shared__ int shm[3 * kWaves];
  __shared__ unsigned long long shu[kWaves];
  const int b = (int)(blockIdx.x / (unsigned)p.C);
  const int j = (int)(blockIdx.x - (unsigned)b * (unsigned)p.C);
  const int64_t l0 = (int64_t)j * kPosChunk + (int64_t)threadIdx.x * kPer;
  Run r;
  read_run(p, b, l0, r);
  // latest valid type before this run in the chunk; the block total is the
  // chunk's last valid type
  // One round: the latest valid type before this run in the chunk (its block
  // total is the chunk's last valid type), the chunk's first valid type (the
  // smallest thread with a valid token), and the bad-type flags.
  const int v1[3] = {r.lt >= 0 ? (int)(threadIdx.x << 2) | r.lt : -1,
                     r.ft >= 0 ? (int)((kPT - 1 - threadIdx.x) << 2) | r.ft : -1, r.flags};
  const int id1[3] = {-1, -1, 0};
  const int kd1[3] = {kScanMax, kScanMax, kScanOr};
  int ex1[3], tot1[3];
  block_scan_multi(v1, id1, kd1, ex1, tot1, shm);
  const int pe = ex1[0], last_enc = tot1[0], first_enc = tot1[1], fl_tot = tot1[2];
  const int pt = pe >= 0 ? (pe & 3) : -1;
  // The run's first valid token starts a segment when a valid token earlier
  // in the chunk has another type; the chunk's first valid token is decided
  // by the carry pass.
  const bool fs = r.ft >= 0 && pt >= 0 && r.ft != pt;
  const int ni = r.ni + (fs && r.ft == 1);
  const int nvd = r.nvd + (fs && r.ft == 2);
  unsigned long long tot;
  const unsigned long long ex = block_excl_sum(pack4(r.nv, r.nt, ni, nvd), &tot, shu);
  const int nv_ex = field(ex, 0);
  // last start of the chunk (chunk-local filtered index, type)
  int cand = -1;
  if (r.lsF >= 0) cand = ((nv_ex + r.lsF) << 2) | r.lsT;
  else if (fs) cand = (nv_ex << 2) | r.ft;
  int last_start;
  block_excl_max(cand, -1, &last_start, sh);
  if (threadIdx.x == 0) {
    // starting values for the fused pass 2+3 (the carry pass rewrites both)
    if (j == 0) p.rope_delta[b] = INT32_MIN;
    if (blockIdx.x == 0) *p.status = 0;
    int* s = p.ws_sum + ((int64_t)b * p.C + j) * kPosSumInts;
    s[0] = field(tot, 0);
    s[1] = field(tot, 1);
    s[2] = field(tot, 2);
    s[3] = field(tot, 3);
    s[4] = first_enc >= 0 ? (first_enc & 3) : -1;
    s[5] = last_enc >= 0 ? (last_enc & 3) : -1;
    s[6] = last_start >= 0 ? (last_start >> 2) : -1;
    s[7] = last_start >= 0 ? (last_start & 3) : -1;
    s[8] = fl_tot;
  }
}

// ---------------------------------------------------------------------------
// Grid helpers (tables built by the carry pass; global memory or an LDS copy).
// ---------------------------------------------------------------------------

struct Tables {
  const int32_t* img;     // [n_images][3]
  const int64_t* adv_i;   // [n_images + 1] image advances before k
  const int32_t* vid;     // [n_videos][3]
  const int32_t* cum_t;   // [n_videos + 1] slices before video v
  const int64_t* adv_v;   // [n_videos + 1] their advances
  int n_images, n_videos, merge;
};

__device__ __forceinline__ Tables global_tables(const RopeIndexParams& p) {
  return Tables{p.image_grid, p.ws_adv_i, p.video_grid, p.ws_cum_t, p.ws_adv_v,
                p.n_images, p.n_videos, p.merge};
}

struct Grid {
  int t, hm, wm, adv;   // slot grid and the advance max(h, w) / merge
  int slots;            // t * hm * wm (grids with 2^31 slots or more are not usable)
  int plane;            // hm * wm
  bool ok;
};

__device__ __forceinline__ int video_of_slice(const Tables& tb, int k) {
  // largest v with cum_t[v] <= k, for 0 <= k < cum_t[n_videos]
  int lo = 0, hi = tb.n_videos - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tb.cum_t[mid] <= k) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Grid of the k-th segment of type `ty` (1 image, 2 video slice).
__device__ Grid grid_of(const Tables& tb, int ty, int k) {
  Grid g;
  g.ok = false;
  g.t = g.hm = g.wm = g.adv = 0;
  g.slots = 0;
  g.plane = 1;
  int t, h, w;
  if (ty == 1) {
    if (k < 0 || k >= tb.n_images) return g;
    t = tb.img[3 * k];
    h = tb.img[3 * k + 1];
    w = tb.img[3 * k + 2];
  } else {
    if (k < 0 || k >= tb.cum_t[tb.n_videos]) return g;
    const int v = video_of_slice(tb, k);
    t = 1;
    h = tb.vid[3 * v + 1];
    w = tb.vid[3 * v + 2];
  }
  g.t = t;
  g.hm = h / tb.merge;
  g.wm = w / tb.merge;
  g.adv = (h > w ? h : w) / tb.merge;
  const int64_t slots = (int64_t)t * g.hm * g.wm;
  g.ok = t > 0 && g.hm > 0 && g.wm > 0 && slots <= INT32_MAX;
  g.slots = g.ok ? (int)slots : 0;
  g.plane = g.ok ? g.hm * g.wm : 1;
  return g;
}

// Sum of the advances of image grids [0, k) and video slices [0, k).
__device__ __forceinline__ int64_t image_adv_before(const Tables& tb, int k) {
  k = k < tb.n_images ? k : tb.n_images;
  return tb.adv_i[k];
}

__device__ __forceinline__ int64_t video_adv_before(const Tables& tb, int k) {
  const int n = tb.cum_t[tb.n_videos];
  k = k < n ? k : n;
  if (k <= 0) return 0;
  if (k == n) return tb.adv_v[tb.n_videos];
  const int v = video_of_slice(tb, k);
  const int h = tb.vid[3 * v + 1], w = tb.vid[3 * v + 2];
  return tb.adv_v[v] + (int64_t)(k - tb.cum_t[v]) * ((h > w ? h : w) / tb.merge);
}

// ---------------------------------------------------------------------------
// Pass 2: grid tables and chunk carries.
//
// The carry of chunk c is a scan over the chunks before it.  Per-sample
// quantities restart at each sample's first chunk b*C; they are taken as the
// batch-wide prefix at c minus the prefix at b*C.  Each thread owns a
// contiguous range of chunks; block scans combine the ranges in three passes
// (valid/text counts and the latest valid type; segment starts by type and
// the latest start; the sample bases), with provisional per-chunk records in
// the summary slots between passes.  Batch-wide filtered indices are below
// 2^29 (checked on the host), so (index << 2 | type) fits an int.
//
// This work is written once, as device functions.  rope_index_carry runs it
// in one block and stores every chunk's carry for rope_index_apply.  When the
// chunk records fit LDS and the grids fit the apply pass's LDS tables,
// rope_index_fused runs it in every block of the apply pass instead and keeps
// its own chunk's carry: one kernel fewer, the same results.
// ---------------------------------------------------------------------------

constexpr int kRecIt = (kPosCarryLds * kPosSumInts + kPT - 1) / kPT;
constexpr int kGridIt = (3 * kPosStageGrids + kPT - 1) / kPT;
constexpr int kAdvIt = (kPosStageGrids + 1 + kPT - 1) / kPT;

// This thread's words of the n chunk summaries (loads issued together).
__device__ __forceinline__ void load_records(const RopeIndexParams& p, int n, int (&rv)[kRecIt]) {
#pragma unroll
  for (int u = 0; u < kRecIt; ++u) {
    const int i = threadIdx.x + u * kPT;
    rv[u] = i < n * kPosSumInts ? p.ws_sum[i] : 0;
  }
}

__device__ __forceinline__ void store_records(const int (&rv)[kRecIt], int n, int* rec) {
#pragma unroll
  for (int u = 0; u < kRecIt; ++u) {
    const int i = threadIdx.x + u * kPT;
    if (i < n * kPosSumInts) rec[i] = rv[u];
  }
}

// Grid-advance prefix tables: adv_i[k] = sum of image advances before k;
// cum_t[v] = slices before video v; adv_v[v] = their advances.  The grids of
// the first tile come in as (ih, iw) and (vt, vh, vw); put(0, k, adv_i[k]),
// put(1, v, cum_t[v]) and put(2, v, adv_v[v]) store the entries.  Returns
// the number of video slices.
// `shl` holds 2 * kWaves entries.
template <typename Put>
__device__ int grid_prefix_tables(const RopeIndexParams& p, int ih, int iw, int vt, int vh,
                                  int vw, long long* shl, Put put) {
  long long carry = 0;
  for (int base = 0; base < p.n_images; base += kPT) {
    const int k = base + threadIdx.x;
    long long a = 0;
    if (k < p.n_images) {
      const int h = base == 0 ? ih : p.image_grid[3 * k + 1];
      const int w = base == 0 ? iw : p.image_grid[3 * k + 2];
      a = (h > w ? h : w) / p.merge;
    }
    long long tot;
    const long long ex = block_excl_sum(a, &tot, shl);
    if (k < p.n_images) put(0, k, carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) put(0, p.n_images, carry);
  long long ct = 0, ca = 0;
  for (int base = 0; base < p.n_videos; base += kPT) {
    const int v = base + threadIdx.x;
    long long t = 0, a = 0;
    if (v < p.n_videos) {
      t = base == 0 ? vt : p.video_grid[3 * v];
      const int h = base == 0 ? vh : p.video_grid[3 * v + 1];
      const int w = base == 0 ? vw : p.video_grid[3 * v + 2];
      t = t > 0 ? t : 0;
      a = t * ((h > w ? h : w) / p.merge);
    }
    const long long v2[2] = {t, a};
    const long long id2[2] = {0, 0};
    const int kd2[2] = {kScanSum, kScanSum};
    long long ex2[2], tot2[2];
    block_scan_multi(v2, id2, kd2, ex2, tot2, shl);
    const long long et = ex2[0], ea = ex2[1], tt = tot2[0], ta = tot2[1];
    if (v < p.n_videos) {
      put(1, v, ct + et);
      put(2, v, ca + ea);
    }
    ct += tt;
    ca += ta;
  }
  if (threadIdx.x == 0) {
    put(1, p.n_videos, ct);
    put(2, p.n_videos, ca);
  }
  return (int)ct;
}

// Carries of the n chunks whose summaries rec holds (overwritten with
// provisional records); `sh` holds 4 * kWaves ints.  emit(c, o) receives chunk c's carry-in;
// end(b, valid, open_len, open_type, open_grid) the end of sample b (its
// valid length and the segment open there).  Returns the status bits the
// summaries report; img_total / vid_total receive the batch's image and video
// segment counts.
template <typename Emit, typename End>
__device__ int chunk_carries(const RopeIndexParams& p, int* rec, int n, int* sh, int* img_total,
                             int* vid_total, Emit emit, End end) {
  const int per = (n + kPT - 1) / kPT;
  const int c0 = min(n, (int)threadIdx.x * per);
  const int c1 = min(n, c0 + per);
  const int C = p.C > 0 ? p.C : 1;

  // Pass 1: valid / text counts, the latest valid type, summary flags.
  int t_nv = 0, t_nt = 0, t_lt = -1, t_flags = 0;
  for (int c = c0; c < c1; ++c) {
    const int* s = rec + (int64_t)c * kPosSumInts;
    t_nv += s[0];
    t_nt += s[1];
    if (s[5] >= 0) t_lt = (c << 2) | s[5];
    t_flags |= s[8];
  }
  const int v1[4] = {t_nv, t_nt, t_lt, t_flags};
  const int id1[4] = {0, 0, -1, 0};
  const int kd1[4] = {kScanSum, kScanSum, kScanMax, kScanOr};
  int ex1[4], tot1[4];
  block_scan_multi(v1, id1, kd1, ex1, tot1, sh);
  int gF = ex1[0], gA = ex1[1], lt = ex1[2];
  const int flags = tot1[3];

  // Pass 2: segment starts (the first valid token of a chunk starts a
  // segment when the latest valid type before it in its sample differs).
  int t_ni = 0, t_nvd = 0, t_st = -1;
  {
    int b = c0 / C, first = b * C;
    for (int c = c0; c < c1; ++c) {
      if (c - first >= C) {
        ++b;
        first += C;
      }
      int* s = rec + (int64_t)c * kPosSumInts;
      const int nv = s[0], nt = s[1], ni = s[2], nvd = s[3], ft = s[4], lts = s[5];
      const int lsF = s[6], lsT = s[7];
      const int prevT = (lt >= 0 && (lt >> 2) >= first) ? (lt & 3) : -1;
      const bool fs = ft >= 0 && ft != prevT;
      const int ni_all = ni + (fs && ft == 1);
      const int nvd_all = nvd + (fs && ft == 2);
      const int cand = lsF >= 0 ? ((gF + lsF) << 2) | lsT : (fs ? (gF << 2) | ft : -1);
      // provisional record (the summary is not needed any more)
      s[0] = gF;
      s[1] = gA;
      s[2] = prevT;
      s[3] = ni_all;
      s[4] = nvd_all;
      s[5] = cand;
      s[8] = nv;
      t_ni += ni_all;
      t_nvd += nvd_all;
      if (cand > t_st) t_st = cand;
      gF += nv;
      gA += nt;
      if (lts >= 0) lt = (c << 2) | lts;
    }
  }
  const int v2[3] = {t_ni, t_nvd, t_st};
  const int id2[3] = {0, 0, -1};
  const int kd2[3] = {kScanSum, kScanSum, kScanMax};
  int ex2[3], tot2[3];
  block_scan_multi(v2, id2, kd2, ex2, tot2, sh);
  int img = ex2[0], vid = ex2[1], st = ex2[2];
  *img_total = tot2[0];
  *vid_total = tot2[1];

  // Pass 3a: grid counters per chunk.
  for (int c = c0; c < c1; ++c) {
    int* s = rec + (int64_t)c * kPosSumInts;
    s[6] = img;
    s[7] = vid;
    img += s[3];
    vid += s[4];
  }
  __threadfence_block();
  __syncthreads();

  // Pass 3b: carries relative to each sample's first chunk.
  {
    int b = c0 / C, first = b * C;
    for (int c = c0; c < c1; ++c) {
      if (c - first >= C) {
        ++b;
        first += C;
      }
      const int* s = rec + (int64_t)c * kPosSumInts;
      const int* s0 = rec + (int64_t)first * kPosSumInts;
      const int F0 = s0[0];
      const int S_in = (st >= 0 && (st >> 2) >= F0) ? (st >> 2) - F0 : -1;
      const int segT_in = S_in >= 0 ? (st & 3) : -1;
      const int o[kPosCarryInts] = {s[0] - F0, s[1] - s0[1], s[2],  s[6],   s[7],
                                    s0[6],     s0[7],       S_in, segT_in};
      emit(c, o);
      if (s[5] > st) st = s[5];
      if (c - first == C - 1) {
        // the sample's end: valid length and the open segment
        const int valid = s[0] + s[8] - F0;
        const int S_end = (st >= 0 && (st >> 2) >= F0) ? (st >> 2) - F0 : -1;
        const int segT_end = S_end >= 0 ? (st & 3) : -1;
        end(b, valid, valid - S_end, segT_end,
            segT_end == 1 ? s[6] + s[3] - 1 : s[7] + s[4] - 1);
      }
    }
  }
  return flags;
}

__global__ void __launch_bounds__(kPT) rope_index_carry(const RopeIndexParams p) {
  __shared__ int sh[4 * kWaves];
  __shared__ long long shl[2 * kWaves];
  __shared__ int rec_lds[kPosCarryLds * kPosSumInts];
  const int n = p.B * p.C;
  // The first tile of each grid table and the chunk records (when they fit
  // LDS) are loaded before any of them is used: one memory round trip.
  const bool rec_in_lds = n <= kPosCarryLds;
  const int tg = 3 * (int)threadIdx.x;
  const int ih = load_in_range(p.image_grid, 3u * (uint32_t)p.n_images, tg + 1);
  const int iw = load_in_range(p.image_grid, 3u * (uint32_t)p.n_images, tg + 2);
  const int vt = load_in_range(p.video_grid, 3u * (uint32_t)p.n_videos, tg);
  const int vh = load_in_range(p.video_grid, 3u * (uint32_t)p.n_videos, tg + 1);
  const int vw = load_in_range(p.video_grid, 3u * (uint32_t)p.n_videos, tg + 2);
  int rv[kRecIt];
  if (rec_in_lds) load_records(p, n, rv);
  const int slices =
      grid_prefix_tables(p, ih, iw, vt, vh, vw, shl, [&](int table, int i, long long v) {
        if (table == 0) p.ws_adv_i[i] = v;
        else if (table == 1) p.ws_cum_t[i] = (int)v;
        else p.ws_adv_v[i] = v;
      });
  // The passes re-read the per-chunk records several times: keep them in LDS
  // when they fit (the provisional records never go back to memory).
  int* const rec = rec_in_lds ? rec_lds : p.ws_sum;
  if (rec_in_lds) {
    store_records(rv, n, rec_lds);
    __syncthreads();
  }
  int img_total, vid_total;
  const int flags = chunk_carries(
      p, rec, n, sh, &img_total, &vid_total,
      [&](int c, const int (&o)[kPosCarryInts]) {
        int* d = p.ws_carry + (int64_t)c * kPosCarryInts;
#pragma unroll
        for (int i = 0; i < kPosCarryInts; ++i) d[i] = o[i];
      },
      [&](int b, int valid, int open_len, int open_type, int open_grid) {
        p.ws_valid[b] = valid;
        p.rope_delta[b] = valid == 0 ? 0 : INT32_MIN;
        int* e = p.ws_end + 3 * b;
        e[0] = open_len;
        e[1] = open_type;
        e[2] = open_grid;
      });
  if (p.C == 0)   // empty sequences: every sample has delta 0
    for (int b = threadIdx.x; b < p.B; b += kPT) p.rope_delta[b] = 0;
  // (each sample's last segment is checked by the apply pass, which has
  // the grid tables at hand)
  if (threadIdx.x == 0) {
    int status = flags;
    if (img_total > p.n_images || vid_total > slices) status |= MROPE_POS_NO_GRID;
    *p.status = status;
  }
}

// ---------------------------------------------------------------------------
// Pass 3: positions.
// ---------------------------------------------------------------------------

// Positions of chunk j of sample b from its carry-in cin, the sample's valid
// length, the segment open at the sample's end e (length, type, grid index;
// read by the sample's last chunk), and the chunk's token words.
// extra_flags are status bits found before; every block ORs its bits into
// the status word and raises rope_delta[b] to its largest position + 1 -
// valid length.  `sh` and `shu` hold kWaves entries, `shl` 2 * kWaves.
__device__ __forceinline__ void apply_chunk(const RopeIndexParams& p, const Tables& tb, int b,
                                            int j, const int (&cin)[kPosCarryInts],
                                            int valid_len, const int* e, const RunWords& words,
                                            int extra_flags, int* sh, unsigned long long* shu,
                                            long long* shl) {
  const int F_in = cin[0], A_in = cin[1], prevT_in = cin[2], img_in = cin[3], vid_in = cin[4];
  const int img_base = cin[5], vid_base = cin[6], S_in = cin[7], segT_in = cin[8];
  const int64_t l0 = (int64_t)j * kPosChunk + (int64_t)threadIdx.x * kPer;
  Run r;
  parse_run(p, l0, words, r);
  int lt_tot;
  const int pe = block_excl_max(r.lt >= 0 ? (int)(threadIdx.x << 2) | r.lt : -1, -1, &lt_tot, sh);
  int prevT = pe >= 0 ? (pe & 3) : prevT_in;
  const bool fs = r.ft >= 0 && r.ft != prevT;
  const int ni = r.ni + (fs && r.ft == 1);
  const int nvd = r.nvd + (fs && r.ft == 2);
  unsigned long long tot;
  const unsigned long long ex = block_excl_sum(pack4(r.nv, r.nt, ni, nvd), &tot, shu);
  int F = F_in + field(ex, 0);
  int A = A_in + field(ex, 1);
  int img = img_in + field(ex, 2);
  int vid = vid_in + field(ex, 3);
  // latest segment start before the run (filtered index << 2 | type)
  int cand = -1;
  if (r.lsF >= 0) cand = ((F + r.lsF) << 2) | r.lsT;
  else if (fs) cand = (F << 2) | r.ft;
  int ctot;
  const int before = block_excl_max(cand, -1, &ctot, sh);
  int S = before >= 0 ? (before >> 2) : S_in;
  int segT = before >= 0 ? (before & 3) : segT_in;

  // the segment open at the start of the run
  Grid g = {0, 0, 0, 0, 0, 1, false};
  if (segT == 1 || segT == 2) g = grid_of(tb, segT, (segT == 1 ? img : vid) - 1);
  const int64_t adv0 = image_adv_before(tb, img_base) + video_adv_before(tb, vid_base);
  int64_t badv = image_adv_before(tb, img) + video_adv_before(tb, vid) - adv0;

  int flags = extra_flags;
  int64_t mx = INT64_MIN;
  const int64_t tok0 = (int64_t)b * p.L + l0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (l0 + k >= p.L) break;
    const int ty = r.ty[k];
    int64_t pt = 0, ph = 0, pw = 0;
    if (ty >= 0) {
      if (ty != prevT) {
        if ((segT == 1 || segT == 2) && g.ok && F - S != g.slots)
          flags |= MROPE_POS_LENGTH;
        S = F;
        segT = ty;
        if (ty == 1) ++img;
        if (ty == 2) ++vid;
        if (ty != 0) {
          g = grid_of(tb, ty, (ty == 1 ? img : vid) - 1);
          badv = image_adv_before(tb, img) + video_adv_before(tb, vid) - adv0;
        }
      }
      prevT = ty;
      if (ty == 0 || !g.ok) {
        if (ty != 0) flags |= MROPE_POS_NO_GRID;
        pt = ph = pw = (int64_t)A + badv;
      } else {
        int i = F - S;
        if (i >= g.slots) {
          flags |= MROPE_POS_LENGTH;
          i = g.slots - 1;
        }
        const int64_t base = (int64_t)A + badv - g.adv;
        const unsigned tt = (unsigned)i / (unsigned)g.plane;
        const unsigned rem = (unsigned)i - tt * (unsigned)g.plane;
        const unsigned row = rem / (unsigned)g.wm;
        pt = base + tt;
        ph = base + row;
        pw = base + (rem - row * (unsigned)g.wm);
      }
      A += ty == 0;
      ++F;
      int64_t m = pt > ph ? pt : ph;
      m = m > pw ? m : pw;
      mx = m > mx ? m : mx;
    }
    const int64_t o = tok0 + k;
    p.pos[o] = (int32_t)pt;
    p.pos[p.pos_stride + o] = (int32_t)ph;
    p.pos[2 * p.pos_stride + o] = (int32_t)pw;
  }
  // the sample's last segment must be complete (checked once, by the block
  // of its last chunk)
  if (j == p.C - 1 && threadIdx.x == 0) {
    if (e[1] == 1 || e[1] == 2) {
      const Grid ge = grid_of(tb, e[1], e[2]);
      if (ge.ok && e[0] != ge.slots) flags |= MROPE_POS_LENGTH;
    }
  }
  const long long v3[2] = {(long long)mx, (long long)flags};
  const long long id3[2] = {(long long)INT64_MIN, 0};
  const int kd3[2] = {kScanMax, kScanOr};
  long long ex3[2], tot3[2];
  block_scan_multi(v3, id3, kd3, ex3, tot3, shl);
  const long long bmax = tot3[0];
  const int f = (int)tot3[1];
  if (threadIdx.x == 0) {
    if (bmax != (long long)INT64_MIN) atomicMax(&p.rope_delta[b], (int)(bmax + 1 - valid_len));
    if (f) atomicOr(p.status, f);
  }
}

__global__ void __launch_bounds__(kPT) rope_index_apply(const RopeIndexParams p) {
  __shared__ int sh[kWaves];
  __shared__ unsigned long long shu[kWaves];
  __shared__ long long shl[2 * kWaves];
  // LDS copy of the grid tables when they are small (the common case): the
  // segment starts of a chunk then look grids up without memory round trips.
  __shared__ int32_t t_img[3 * kPosStageGrids];
  __shared__ int64_t t_adv_i[kPosStageGrids + 1];
  __shared__ int32_t t_vid[3 * kPosStageGrids];
  __shared__ int32_t t_cum_t[kPosStageGrids + 1];
  __shared__ int64_t t_adv_v[kPosStageGrids + 1];
  // Every global load of the block (the tables, the chunk's carry, its
  // tokens) is issued before the first wait, so the block pays one memory
  // round trip before its scans.
  Tables tb = global_tables(p);
  const bool stage = p.n_images <= kPosStageGrids && p.n_videos <= kPosStageGrids;
  int32_t gi[kGridIt], gv[kGridIt], gc[kAdvIt];
  int64_t ga[kAdvIt], gw[kAdvIt];
  if (stage) {
#pragma unroll
    for (int u = 0; u < kGridIt; ++u) {
      const int i = threadIdx.x + u * kPT;
      gi[u] = i < 3 * p.n_images ? p.image_grid[i] : 0;
      gv[u] = i < 3 * p.n_videos ? p.video_grid[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kAdvIt; ++u) {
      const int i = threadIdx.x + u * kPT;
      ga[u] = i <= p.n_images ? p.ws_adv_i[i] : 0;
      gc[u] = i <= p.n_videos ? p.ws_cum_t[i] : 0;
      gw[u] = i <= p.n_videos ? p.ws_adv_v[i] : 0;
    }
  }
  const int b = (int)(blockIdx.x / (unsigned)p.C);
  const int j = (int)(blockIdx.x - (unsigned)b * (unsigned)p.C);
  int cin[kPosCarryInts];
  const int* cg = p.ws_carry + ((int64_t)b * p.C + j) * kPosCarryInts;
#pragma unroll
  for (int i = 0; i < kPosCarryInts; ++i) cin[i] = cg[i];
  const int valid_len = p.ws_valid[b];

  const int64_t l0 = (int64_t)j * kPosChunk + (int64_t)threadIdx.x * kPer;
  RunWords words;
  load_run(p, b, l0, words);
  if (stage) {
#pragma unroll
    for (int u = 0; u < kGridIt; ++u) {
      const int i = threadIdx.x + u * kPT;
      if (i < 3 * p.n_images) t_img[i] = gi[u];
      if (i < 3 * p.n_videos) t_vid[i] = gv[u];
    }
#pragma unroll
    for (int u = 0; u < kAdvIt; ++u) {
      const int i = threadIdx.x + u * kPT;
      if (i <= p.n_images) t_adv_i[i] = ga[u];
      if (i <= p.n_videos) {
        t_cum_t[i] = gc[u];
        t_adv_v[i] = gw[u];
      }
    }
    tb.img = t_img;
    tb.adv_i = t_adv_i;
    tb.vid = t_vid;
    tb.cum_t = t_cum_t;
    tb.adv_v = t_adv_v;
    // the copies are ordered before their first use by the barriers of the
    // block scans in apply_chunk
  }
  // bad types were reported by the summary pass, through the carry pass
  apply_chunk(p, tb, b, j, cin, valid_len, p.ws_end + 3 * b, words, 0, sh, shu, shl);
}

// Passes 2 and 3 in one kernel (the chunk records fit LDS, the grids fit the
// LDS tables): each block runs the carry work on the whole batch in LDS and
// then writes its own chunk's positions.  The summary pass has set the
// status word to 0 and every rope_delta to INT32_MIN.
__global__ void __launch_bounds__(kPT) rope_index_fused(const RopeIndexParams p) {
  __shared__ int sh[4 * kWaves];
  __shared__ unsigned long long shu[kWaves];
  __shared__ long long shl[2 * kWaves];
  __shared__ int rec_lds[kPosCarryLds * kPosSumInts];
  __shared__ int32_t t_img[3 * kPosStageGrids];
  __shared__ int64_t t_adv_i[kPosStageGrids + 1];
  __shared__ int32_t t_vid[3 * kPosStageGrids];
  __shared__ int32_t t_cum_t[kPosStageGrids + 1];
  __shared__ int64_t t_adv_v[kPosStageGrids + 1];
  __shared__ int own_carry[kPosCarryInts];
  __shared__ int own_end[4];   // valid length, open length, open type, open grid
  const int n = p.B * p.C;
  const int b = (int)(blockIdx.x / (unsigned)p.C);
  const int j = (int)(blockIdx.x - (unsigned)b * (unsigned)p.C);
  const int c_self = (int)blockIdx.x;
  // every global load first: grids, chunk summaries, this chunk's tokens
  int32_t gi[kGridIt], gv[kGridIt];
#pragma unroll
  for (int u = 0; u < kGridIt; ++u) {
    const int i = threadIdx.x + u * kPT;
    gi[u] = load_in_range(p.image_grid, 3u * (uint32_t)p.n_images, i);
    gv[u] = load_in_range(p.video_grid, 3u * (uint32_t)p.n_videos, i);
  }
  int rv[kRecIt];
  load_records(p, n, rv);
  const int64_t l0 = (int64_t)j * kPosChunk + (int64_t)threadIdx.x * kPer;
  RunWords words;
  load_run(p, b, l0, words);
#pragma unroll
  for (int u = 0; u < kGridIt; ++u) {
    const int i = threadIdx.x + u * kPT;
    if (i < 3 * p.n_images) t_img[i] = gi[u];
    if (i < 3 * p.n_videos) t_vid[i] = gv[u];
  }
  store_records(rv, n, rec_lds);
  __syncthreads();
  const int k = threadIdx.x;
  const int ih = k < p.n_images ? t_img[3 * k + 1] : 0;
  const int iw = k < p.n_images ? t_img[3 * k + 2] : 0;
  const int vt = k < p.n_videos ? t_vid[3 * k] : 0;
  const int vh = k < p.n_videos ? t_vid[3 * k + 1] : 0;
  const int vw = k < p.n_videos ? t_vid[3 * k + 2] : 0;
  const int slices =
      grid_prefix_tables(p, ih, iw, vt, vh, vw, shl, [&](int table, int i, long long v) {
        if (table == 0) t_adv_i[i] = v;
        else if (table == 1) t_cum_t[i] = (int)v;
        else t_adv_v[i] = v;
      });
  int img_total, vid_total;
  int flags = chunk_carries(
      p, rec_lds, n, sh, &img_total, &vid_total,
      [&](int c, const int (&o)[kPosCarryInts]) {
        if (c == c_self) {
#pragma unroll
          for (int i = 0; i < kPosCarryInts; ++i) own_carry[i] = o[i];
        }
      },
      [&](int bb, int valid, int open_len, int open_type, int open_grid) {
        if (bb == b) {
          own_end[0] = valid;
          own_end[1] = open_len;
          own_end[2] = open_type;
          own_end[3] = open_grid;
        }
      });
  if (img_total > p.n_images || vid_total > slices) flags |= MROPE_POS_NO_GRID;
  __syncthreads();
  int cin[kPosCarryInts];
#pragma unroll
  for (int i = 0; i < kPosCarryInts; ++i) cin[i] = own_carry[i];
  const int valid_len = own_end[0];
  // a sample without valid tokens raises no rope_delta: its delta is 0
  if (valid_len == 0 && j == p.C - 1 && threadIdx.x == 0) p.rope_delta[b] = 0;
  const Tables tb{t_img, t_adv_i, t_vid, t_cum_t, t_adv_v, p.n_images, p.n_videos, p.merge};
  apply_chunk(p, tb, b, j, cin, valid_len, own_end + 1, words, flags, sh, shu, shl);
}

// ---------------------------------------------------------------------------
// Vision patch coordinates.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(kPT) vision_pos_ids_kernel(const VisionPosParams p) {
  extern __shared__ long long cum[];   // n_images + 1 patch-count prefix
  __shared__ long long shl[kWaves];
  __shared__ int sh[kWaves];
  int bad = 0;
  long long carry = 0;
  for (int base = 0; base < p.n_images; base += kPT) {
    const int k = base + threadIdx.x;
    long long n = 0;
    if (k < p.n_images) {
      const int t = p.grid[3 * k], h = p.grid[3 * k + 1], w = p.grid[3 * k + 2];
      if (t < 0 || h < 0 || w < 0) bad = 1;
      else n = (long long)t * h * w;
      if (h % p.merge != 0 || w % p.merge != 0) bad = 1;
    }
    long long tot;
    const long long ex = block_excl_sum(n, &tot, shl);
    if (k < p.n_images) cum[k] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) cum[p.n_images] = carry;
  const int any_bad = block_or(bad, sh);
  __syncthreads();
  const long long total = cum[p.n_images];
  if (blockIdx.x == 0 && threadIdx.x == 0)
    *p.status = (any_bad ? MROPE_POS_NOT_DIVISIBLE : 0) | (total != p.N ? MROPE_POS_COUNT : 0);

  const int m = p.merge;
  for (int64_t idx = (int64_t)blockIdx.x * kPT + threadIdx.x; idx < p.N;
       idx += (int64_t)gridDim.x * kPT) {
    int32_t row = 0, col = 0;
    if (idx < total) {
      int lo = 0, hi = p.n_images - 1;   // last image with cum <= idx
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cum[mid] <= idx) lo = mid;
        else hi = mid - 1;
      }
      const int h = p.grid[3 * lo + 1], w = p.grid[3 * lo + 2];
      const int64_t frame = (int64_t)h * w;
      const int64_t jj = (idx - cum[lo]) % frame;
      const int wm = w / m;
      const int64_t blk = jj / (m * m);
      const int intra = (int)(jj - blk * m * m);
      const int64_t by = wm > 0 ? blk / wm : 0;
      const int64_t bx = blk - by * wm;
      row = (int32_t)(by * m + intra / m);
      col = (int32_t)(bx * m + intra % m);
    }
    p.pos[idx] = row;
    p.pos[p.pos_stride + idx] = col;
  }
}

}  // namespace

int launch_rope_index(const RopeIndexParams& p, void* stream, const char** kernel) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t chunks = (int64_t)p.B * p.C;
  if (chunks > 0)
    hipLaunchKernelGGL(rope_index_summarize, dim3((unsigned)chunks), dim3(kPT), 0, st, p);
  const bool fused = chunks > 0 && chunks <= kPosCarryLds && p.n_images <= kPosStageGrids &&
                     p.n_videos <= kPosStageGrids;
  *kernel = fused ? "rope_index_fused" : "rope_index_carry+apply";
  if (fused) {
    hipLaunchKernelGGL(rope_index_fused, dim3((unsigned)chunks), dim3(kPT), 0, st, p);
  } else {
    hipLaunchKernelGGL(rope_index_carry, dim3(1), dim3(kPT), 0, st, p);
    if (chunks > 0)
      hipLaunchKernelGGL(rope_index_apply, dim3((unsigned)chunks), dim3(kPT), 0, st, p);
  }
  return (int)hipGetLastError();
}

int launch_vision_pos_ids(const VisionPosParams& p, void* stream) {
  int64_t blocks = (p.N + kPT - 1) / kPT;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  const size_t lds = (size_t)(p.n_images + 1) * sizeof(long long);
  hipLaunchKernelGGL(vision_pos_ids_kernel, dim3((unsigned)blocks), dim3(kPT), lds,
                     static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

}  // namespace mrope
