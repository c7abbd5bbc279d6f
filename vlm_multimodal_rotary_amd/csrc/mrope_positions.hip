// Position builders for multimodal rotary embedding on gfx950.
//
// rope_index: the 3-axis (T, H, W) position table of a batch of mixed text /
// image / video token sequences plus the per-sample rope_deltas ("Interleaved
// Rotary Position Embedding", get_rope_index walkthrough).  Every position is
// a prefix quantity of the token sequence, so the builder is three scans:
//
//   1. summarize: one block per 4096-token chunk of a sample reduces the
//      chunk (valid and text token counts, first/last valid type, segment
//      starts by type, the last start) -- tokens are read once.
//   2. carry:     one block walks the chunk summaries in order (in LDS tiles)
//      and writes each chunk's carry-in: filtered index, text count, the
//      previous valid type, the global image / video grid counters, the open
//      segment; it also builds the grid-advance prefix tables and the
//      per-sample valid length.
//   3. apply:     one block per chunk re-reads its tokens, resolves segment
//      starts with block scans seeded by the carry, and writes the positions;
//      rope_delta = max + 1 - valid length by one atomic max per block.
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

#include "mrope_internal.h"

namespace mrope {
namespace {

constexpr int kPT = kPosThreads;
constexpr int kPer = kPosPerThread;
constexpr int kWaves = kPT / kWaveSize;

// ---------------------------------------------------------------------------
// Block scans over 256 threads (four wavefronts).
// ---------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ T wave_incl_sum(T v) {
  const int lane = threadIdx.x & (kWaveSize - 1);
#pragma unroll
  for (int d = 1; d < kWaveSize; d <<= 1) {
    const T u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_incl_max(T v) {
  const int lane = threadIdx.x & (kWaveSize - 1);
#pragma unroll
  for (int d = 1; d < kWaveSize; d <<= 1) {
    const T u = __shfl_up(v, d);
    if (lane >= d && u > v) v = u;
  }
  return v;
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
  const T incl = wave_incl_max(v);
  T prev = __shfl_up(incl, 1);
  if (lane == 0) prev = lo;
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

// Bitwise OR over the block.
__device__ int block_or(int v, int* sh) {
  const int w = threadIdx.x / kWaveSize;
  const int lane = threadIdx.x & (kWaveSize - 1);
#pragma unroll
  for (int d = 1; d < kWaveSize; d <<= 1) v |= __shfl_xor(v, d);
  if (lane == 0) sh[w] = v;
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

__device__ __forceinline__ void read_run(const RopeIndexParams& p, int b, int64_t l0, Run& r) {
  r.nv = r.nt = r.ni = r.nvd = 0;
  r.ft = r.lt = r.lsF = r.lsT = -1;
  r.flags = 0;
  const int64_t row = (int64_t)b * p.L;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t l = l0 + k;
    int ty = -1;
    if (l < p.L) {
      const bool v = p.mask == nullptr || p.mask[row + l] != 0;
      if (v) {
        ty = p.types[row + l];
        if (ty < 0 || ty > 2) {
          r.flags |= MROPE_POS_BAD_TYPE;
          ty = 0;
        }
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

// The latest valid type of the threads before this one in the block, as an
// encoded max: (thread << 2 | type), -1 for none.
__device__ __forceinline__ int prev_type_in_block(const Run& r, int* sh) {
  int tot;
  const int enc = r.lt >= 0 ? (int)(threadIdx.x << 2) | r.lt : -1;
  const int m = block_excl_max(enc, -1, &tot, sh);
  return m >= 0 ? (m & 3) : -1;
}

// ---------------------------------------------------------------------------
// Pass 1: chunk summaries.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(kPT) rope_index_summarize(const RopeIndexParams p) {
  __shared__ int sh[kWaves];
  __shared__ long long shl[kWaves];
  const int b = (int)(blockIdx.x / (unsigned)p.C);
  const int j = (int)(blockIdx.x - (unsigned)b * (unsigned)p.C);
  const int64_t l0 = (int64_t)j * kPosChunk + (int64_t)threadIdx.x * kPer;
  Run r;
  read_run(p, b, l0, r);
  const int pt = prev_type_in_block(r, sh);
  // The run's first valid token starts a segment when a valid token earlier
  // in the chunk has another type; the chunk's first valid token is decided
  // by the carry pass.
  const bool fs = r.ft >= 0 && pt >= 0 && r.ft != pt;
  const int ni = r.ni + (fs && r.ft == 1);
  const int nvd = r.nvd + (fs && r.ft == 2);
  int nv_tot, nt_tot, ni_tot, nvd_tot;
  const int nv_ex = block_excl_sum(r.nv, &nv_tot, sh);
  block_excl_sum(r.nt, &nt_tot, sh);
  block_excl_sum(ni, &ni_tot, sh);
  block_excl_sum(nvd, &nvd_tot, sh);
  const int fl_tot = block_or(r.flags, sh);
  // last start of the chunk (chunk-local filtered index, type)
  long long cand = -1;
  if (r.lsF >= 0) cand = ((long long)(nv_ex + r.lsF) << 2) | r.lsT;
  else if (fs) cand = ((long long)nv_ex << 2) | r.ft;
  long long last_start;
  block_excl_max(cand, -1LL, &last_start, shl);
  // first and last valid type of the chunk
  int first_enc, last_enc;
  block_excl_max(r.ft >= 0 ? (int)((kPT - 1 - threadIdx.x) << 2) | r.ft : -1, -1, &first_enc, sh);
  block_excl_max(r.lt >= 0 ? (int)(threadIdx.x << 2) | r.lt : -1, -1, &last_enc, sh);
  if (threadIdx.x == 0) {
    int* s = p.ws_sum + ((int64_t)b * p.C + j) * kPosSumInts;
    s[0] = nv_tot;
    s[1] = nt_tot;
    s[2] = ni_tot;
    s[3] = nvd_tot;
    s[4] = first_enc >= 0 ? (first_enc & 3) : -1;
    s[5] = last_enc >= 0 ? (last_enc & 3) : -1;
    s[6] = last_start >= 0 ? (int)(last_start >> 2) : -1;
    s[7] = last_start >= 0 ? (int)(last_start & 3) : -1;
    s[8] = fl_tot;
  }
}

// ---------------------------------------------------------------------------
// Grid helpers (tables built by the carry pass).
// ---------------------------------------------------------------------------

struct Grid {
  int t, hm, wm, adv;   // slot grid and the advance max(h, w) / merge
  int64_t slots;
  bool ok;
};

__device__ __forceinline__ int video_of_slice(const RopeIndexParams& p, int k) {
  // largest v with cum_t[v] <= k, for 0 <= k < cum_t[n_videos]
  int lo = 0, hi = p.n_videos - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.ws_cum_t[mid] <= k) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Grid of the k-th segment of type `ty` (1 image, 2 video slice).
__device__ Grid grid_of(const RopeIndexParams& p, int ty, int k) {
  Grid g;
  g.ok = false;
  g.t = g.hm = g.wm = g.adv = 0;
  g.slots = 0;
  int t, h, w;
  if (ty == 1) {
    if (k < 0 || k >= p.n_images) return g;
    t = p.image_grid[3 * k];
    h = p.image_grid[3 * k + 1];
    w = p.image_grid[3 * k + 2];
  } else {
    if (k < 0 || k >= p.ws_cum_t[p.n_videos]) return g;
    const int v = video_of_slice(p, k);
    t = 1;
    h = p.video_grid[3 * v + 1];
    w = p.video_grid[3 * v + 2];
  }
  g.t = t;
  g.hm = h / p.merge;
  g.wm = w / p.merge;
  g.adv = (h > w ? h : w) / p.merge;
  g.slots = (int64_t)t * g.hm * g.wm;
  g.ok = t > 0 && g.hm > 0 && g.wm > 0;
  return g;
}

// Sum of the advances of image grids [0, k) and video slices [0, k).
__device__ __forceinline__ int64_t image_adv_before(const RopeIndexParams& p, int k) {
  k = k < p.n_images ? k : p.n_images;
  return p.ws_adv_i[k];
}

__device__ __forceinline__ int64_t video_adv_before(const RopeIndexParams& p, int k) {
  const int n = p.ws_cum_t[p.n_videos];
  k = k < n ? k : n;
  if (k <= 0) return 0;
  if (k == n) return p.ws_adv_v[p.n_videos];
  const int v = video_of_slice(p, k);
  const int h = p.video_grid[3 * v + 1], w = p.video_grid[3 * v + 2];
  return p.ws_adv_v[v] + (int64_t)(k - p.ws_cum_t[v]) * ((h > w ? h : w) / p.merge);
}

// ---------------------------------------------------------------------------
// Pass 2: grid tables and chunk carries (one block).
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(kPT) rope_index_carry(const RopeIndexParams p) {
  __shared__ long long shl[kWaves];
  __shared__ int tile[kPosCarryTile * kPosSumInts];
  __shared__ int out[kPosCarryTile * kPosCarryInts];
  // Grid-advance prefix tables: adv_i[k] = sum of image advances before k;
  // cum_t[v] = slices before video v; adv_v[v] = their advances.
  long long carry = 0;
  for (int base = 0; base < p.n_images; base += kPT) {
    const int k = base + threadIdx.x;
    long long a = 0;
    if (k < p.n_images) {
      const int h = p.image_grid[3 * k + 1], w = p.image_grid[3 * k + 2];
      a = (h > w ? h : w) / p.merge;
    }
    long long tot;
    const long long ex = block_excl_sum(a, &tot, shl);
    if (k < p.n_images) p.ws_adv_i[k] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) p.ws_adv_i[p.n_images] = carry;
  long long ct = 0, ca = 0;
  for (int base = 0; base < p.n_videos; base += kPT) {
    const int v = base + threadIdx.x;
    long long t = 0, a = 0;
    if (v < p.n_videos) {
      t = p.video_grid[3 * v];
      const int h = p.video_grid[3 * v + 1], w = p.video_grid[3 * v + 2];
      t = t > 0 ? t : 0;
      a = t * ((h > w ? h : w) / p.merge);
    }
    long long tt, ta;
    const long long et = block_excl_sum(t, &tt, shl);
    const long long ea = block_excl_sum(a, &ta, shl);
    if (v < p.n_videos) {
      p.ws_cum_t[v] = (int)(ct + et);
      p.ws_adv_v[v] = ca + ea;
    }
    ct += tt;
    ca += ta;
  }
  if (threadIdx.x == 0) {
    p.ws_cum_t[p.n_videos] = (int)ct;
    p.ws_adv_v[p.n_videos] = ca;
  }
  __threadfence_block();
  __syncthreads();

  // Sequential walk over the chunk summaries, a tile at a time through LDS.
  // State lives in thread 0's registers between tiles.
  int status = 0;
  int img = 0, vid = 0;
  int F = 0, A = 0, prevT = -1, S = -1, segT = -1, img_base = 0, vid_base = 0;
  const int64_t n_chunks = (int64_t)p.B * p.C;
  for (int64_t t0 = 0; t0 < n_chunks; t0 += kPosCarryTile) {
    const int n = (int)((n_chunks - t0) < kPosCarryTile ? (n_chunks - t0) : kPosCarryTile);
    for (int i = threadIdx.x; i < n * kPosSumInts; i += kPT) tile[i] = p.ws_sum[t0 * kPosSumInts + i];
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int i = 0; i < n; ++i) {
        const int64_t c = t0 + i;
        const int b = (int)(c / p.C);
        const int j = (int)(c - (int64_t)b * p.C);
        if (j == 0) {
          F = A = 0;
          prevT = S = segT = -1;
          img_base = img;
          vid_base = vid;
        }
        int* o = out + i * kPosCarryInts;
        o[0] = F;
        o[1] = A;
        o[2] = prevT;
        o[3] = img;
        o[4] = vid;
        o[5] = img_base;
        o[6] = vid_base;
        o[7] = S;
        o[8] = segT;
        const int* s = tile + i * kPosSumInts;
        status |= s[8];
        const bool fs = s[4] >= 0 && s[4] != prevT;
        img += s[2] + (fs && s[4] == 1);
        vid += s[3] + (fs && s[4] == 2);
        if (s[6] >= 0) {
          S = F + s[6];
          segT = s[7];
        } else if (fs) {
          S = F;
          segT = s[4];
        }
        F += s[0];
        A += s[1];
        if (s[5] >= 0) prevT = s[5];
        if (j == p.C - 1) {
          p.ws_valid[b] = F;
          p.rope_delta[b] = F == 0 ? 0 : INT32_MIN;
          // the sample's last segment must be complete
          if (segT == 1 || segT == 2) {
            const Grid g = grid_of(p, segT, (segT == 1 ? img : vid) - 1);
            if (g.ok && (int64_t)(F - S) != g.slots) status |= MROPE_POS_LENGTH;
          }
        }
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n * kPosCarryInts; i += kPT)
      p.ws_carry[t0 * kPosCarryInts + i] = out[i];
    __syncthreads();
  }
  if (p.C == 0)   // empty sequences: every sample has delta 0
    for (int b = threadIdx.x; b < p.B; b += kPT) p.rope_delta[b] = 0;
  if (threadIdx.x == 0) {
    if (img > p.n_images || vid > p.ws_cum_t[p.n_videos]) status |= MROPE_POS_NO_GRID;
    *p.status = status;
  }
}

// ---------------------------------------------------------------------------
// Pass 3: positions.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(kPT) rope_index_apply(const RopeIndexParams p) {
  __shared__ int sh[kWaves];
  __shared__ long long shl[kWaves];
  const int b = (int)(blockIdx.x / (unsigned)p.C);
  const int j = (int)(blockIdx.x - (unsigned)b * (unsigned)p.C);
  const int* cin = p.ws_carry + ((int64_t)b * p.C + j) * kPosCarryInts;
  const int F_in = cin[0], A_in = cin[1], prevT_in = cin[2], img_in = cin[3], vid_in = cin[4];
  const int img_base = cin[5], vid_base = cin[6], S_in = cin[7], segT_in = cin[8];
  const int valid_len = p.ws_valid[b];

  const int64_t l0 = (int64_t)j * kPosChunk + (int64_t)threadIdx.x * kPer;
  Run r;
  read_run(p, b, l0, r);
  const int pt_blk = prev_type_in_block(r, sh);
  int prevT = pt_blk >= 0 ? pt_blk : prevT_in;
  const bool fs = r.ft >= 0 && r.ft != prevT;
  const int ni = r.ni + (fs && r.ft == 1);
  const int nvd = r.nvd + (fs && r.ft == 2);
  int tot;
  int F = F_in + block_excl_sum(r.nv, &tot, sh);
  int A = A_in + block_excl_sum(r.nt, &tot, sh);
  int img = img_in + block_excl_sum(ni, &tot, sh);
  int vid = vid_in + block_excl_sum(nvd, &tot, sh);
  long long cand = -1;
  const int f_run = F;   // filtered index of the run's first valid token
  if (r.lsF >= 0) cand = ((long long)(f_run + r.lsF) << 2) | r.lsT;
  else if (fs) cand = ((long long)f_run << 2) | r.ft;
  long long ltot;
  const long long before = block_excl_max(cand, -1LL, &ltot, shl);
  int S = before >= 0 ? (int)(before >> 2) : S_in;
  int segT = before >= 0 ? (int)(before & 3) : segT_in;

  // the segment open at the start of the run
  Grid g = {0, 0, 0, 0, 0, false};
  if (segT == 1 || segT == 2) g = grid_of(p, segT, (segT == 1 ? img : vid) - 1);
  const int64_t adv_i0 = image_adv_before(p, img_base);
  const int64_t adv_v0 = video_adv_before(p, vid_base);
  int64_t badv = image_adv_before(p, img) - adv_i0 + video_adv_before(p, vid) - adv_v0;

  int flags = 0;   // bad types were reported by the summary pass
  int64_t mx = INT64_MIN;
  const int64_t tok0 = (int64_t)b * p.L + l0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (l0 + k >= p.L) break;
    const int ty = r.ty[k];
    int64_t pt = 0, ph = 0, pw = 0;
    if (ty >= 0) {
      if (ty != prevT) {
        if ((segT == 1 || segT == 2) && g.ok && (int64_t)(F - S) != g.slots)
          flags |= MROPE_POS_LENGTH;
        S = F;
        segT = ty;
        if (ty == 1) ++img;
        if (ty == 2) ++vid;
        if (ty != 0) {
          g = grid_of(p, ty, (ty == 1 ? img : vid) - 1);
          badv = image_adv_before(p, img) - adv_i0 + video_adv_before(p, vid) - adv_v0;
        }
      }
      prevT = ty;
      if (ty == 0 || !g.ok) {
        if (ty != 0) flags |= MROPE_POS_NO_GRID;
        pt = ph = pw = (int64_t)A + badv;
      } else {
        int64_t i = F - S;
        if (i >= g.slots) {
          flags |= MROPE_POS_LENGTH;
          i = g.slots - 1;
        }
        const int64_t base = (int64_t)A + badv - g.adv;
        const int64_t plane = (int64_t)g.hm * g.wm;
        const int64_t tt = i / plane;
        const int64_t rem = i - tt * plane;
        const int64_t row = rem / g.wm;
        pt = base + tt;
        ph = base + row;
        pw = base + (rem - row * g.wm);
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
  long long bmax;
  block_excl_max((long long)mx, (long long)INT64_MIN, &bmax, shl);
  const int f = block_or(flags, sh);
  if (threadIdx.x == 0) {
    if (bmax != (long long)INT64_MIN) atomicMax(&p.rope_delta[b], (int)(bmax + 1 - valid_len));
    if (f) atomicOr(p.status, f);
  }
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

int launch_rope_index(const RopeIndexParams& p, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t chunks = (int64_t)p.B * p.C;
  if (chunks > 0)
    hipLaunchKernelGGL(rope_index_summarize, dim3((unsigned)chunks), dim3(kPT), 0, st, p);
  hipLaunchKernelGGL(rope_index_carry, dim3(1), dim3(kPT), 0, st, p);
  if (chunks > 0)
    hipLaunchKernelGGL(rope_index_apply, dim3((unsigned)chunks), dim3(kPT), 0, st, p);
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
