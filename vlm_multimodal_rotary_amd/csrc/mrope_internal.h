// Internal types shared by the host entry points and the HIP kernels.
#pragma once

#include <stdint.h>

#include "../../include/mrope.h"

namespace mrope {

constexpr int kMaxHalf = MROPE_MAX_ROTARY_DIM / 2;
constexpr int kWaveSize = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWaveSize * kWavesPerBlock;
// Chunks the flat kernel loads before it stores any (six per lane).  A row
// whose halves fall in different batches reads its partner after the first
// batch's stores, so an in-place tensor must fit one batch per token.
constexpr int kFlatBatchChunks = 6 * kWaveSize;

// Per frequency column j < half: the binary32 inverse frequency it multiplies
// and the position axis it reads.  Passed by value as a kernel argument; the
// kernels index it per lane, which the compiler turns into vector loads from
// the kernel-argument segment.
struct ColTable {
  float inv[kMaxHalf];
  uint8_t axis[kMaxHalf];
  uint8_t fidx[kMaxHalf];   // index of inv[j] among the distinct frequencies
};

// How the cos/sin of a row's token are obtained.
enum CsMode : int {
  kCsFromPositions = 0,  // computed per tile from positions (fused path)
  kCsFromTable = 1,      // read from caller cos/sin tables [T][rotary_dim]
  kCsNone = 2,           // no rotation (RMSNorm only)
  kCsDecode = 3,         // decode: text positions from cache length + rope_delta,
                         // k written to a KV cache (one token per wavefront)
};

// One launch processes up to three tensors (slot 0 = q, slot 1 = k, slot 2 =
// v of a packed qkv, copied only) that share T, D, rotary_dim and the
// per-token cos/sin.  Inputs have contiguous heads; outputs have a head
// stride (D for token-major rows, T*D for head-major planes).
constexpr int kSlots = 3;

struct QKParams {
  const void* x[kSlots];
  void* y[kSlots];
  const void* w[kSlots];   // RMSNorm weights (dtype of x) or null
  int64_t x_ts[kSlots];    // token strides, elements
  int64_t y_ts[kSlots];
  int64_t y_hs[kSlots];    // output head strides, elements
  int heads[kSlots];
  int64_t T;
  int D;
  int rd;                // rotary dim (0 for RMSNorm only)
  int half;              // rd / 2
  int lpr;               // lanes per head row: D / (2 * V)
  int rpw;               // rows per wavefront instruction: 64 / lpr
  int lrot;              // rotary lanes per row: half / V
  int nt;                // tokens per tile (set by the launcher)
  int parts;             // wavefronts per tile (set by the launcher)
  int waves_cap;         // resident wavefronts per SIMD at most (0 = no bound)
  float inv_cpr;         // flat kernel: 1 / (D / V); staged kernel: 1 / (D * ES / 16)
  int stage_hm;          // staged kernel: write head-major order (1) or token-major (0)
  int dq[kSlots], dr[kSlots];   // rpw = dq * heads + dr, per tensor (launcher)
  float inv_heads[kSlots];      // 1 / heads, per tensor (launcher)
  float inv_run;                // group kernel: 1 / (nt * D / V), chunks of a plane's run
  const int32_t* pos;
  int64_t pos_stride;
  // axis of frequency column j as a rule (set by the launcher from the
  // column table): ax_mode 0: (j >= ax_a) + (j >= ax_b); 1: 1 if j % 3 == 1
  // and j < ax_a, 2 if j % 3 == 2 and j < ax_b, else 0; -1: read the table
  int ax_mode, ax_a, ax_b;
  const float* cos;
  const float* sin;
  int64_t cs_ts;
  float eps;
  double inv_d;          // 1.0 / D
  // optional cos/sin cache by position: (cos, sin) of fl32(p * inv) at
  // cs_cache[2 * (p * n_freq + fidx[j])], for 0 <= p < cache_rows
  const float* cs_cache;
  int cache_rows;
  int n_freq;
  // decode mode
  const int32_t* cache_len;   // [batch]
  const int32_t* rope_delta;  // [batch] or null
  int new_tokens;             // tokens per sequence; token t = b * new_tokens + i
  int64_t kc_seq;             // k-cache stride between sequences (elements)
  int64_t kc_tok;             // k-cache stride between positions (elements)
  int kc_cap;                 // k-cache positions per sequence
};

struct CosSinParams {
  const int32_t* pos;
  int64_t pos_stride;
  int64_t T;
  int half;
  int rd;
  float* cos;
  float* sin;
  int64_t cs_ts;
};

// Position builders (mrope_positions.hip).
constexpr int kPosThreads = 256;
constexpr int kPosPerThread = 4;
constexpr int kPosChunk = kPosThreads * kPosPerThread;   // tokens per block
constexpr int kPosSumInts = 9;      // chunk summary: nv, nt, ni, nvd, ft, lt, lsF, lsT, flags
constexpr int kPosCarryInts = 9;    // chunk carry: F, A, prevT, img, vid, img0, vid0, S, segT
constexpr int kPosCarryLds = 1024;   // chunk records the carry pass keeps in LDS
constexpr int kPosStageGrids = 256;  // grids per type the apply pass copies to LDS
constexpr int kMaxVisionImages = 4096;   // patch-count prefix in LDS: 32 KB

struct RopeIndexParams {
  const int32_t* types;       // [B][L]
  const int32_t* mask;        // [B][L] or null
  int B;
  int64_t L;
  int C;                      // chunks per sample
  const int32_t* image_grid;  // [n_images][3]
  int n_images;
  const int32_t* video_grid;  // [n_videos][3]
  int n_videos;
  int merge;
  int32_t* pos;               // [3][B*L], axis stride pos_stride
  int64_t pos_stride;
  int32_t* rope_delta;        // [B]
  int32_t* status;
  // workspace regions
  int32_t* ws_sum;            // [B*C][kPosSumInts]
  int32_t* ws_carry;          // [B*C][kPosCarryInts]
  int32_t* ws_valid;          // [B]
  int32_t* ws_end;            // [B][3] open segment at each sample's end
  int64_t* ws_adv_i;          // [n_images + 1]
  int64_t* ws_adv_v;          // [n_videos + 1]
  int32_t* ws_cum_t;          // [n_videos + 1]
};

struct VisionPosParams {
  const int32_t* grid;        // [n_images][3]
  int n_images;
  int merge;
  int64_t N;                  // patches the output holds
  int32_t* pos;               // [2][N], axis stride pos_stride
  int64_t pos_stride;
  int32_t* status;
};

// *kernel receives the name of the pass-2/3 form launched.
int launch_rope_index(const RopeIndexParams& p, void* stream, const char** kernel);
// Bytes of the static workspace of mrope_rope_index_noalloc, and its device
// address on the current device (taken once per device with
// hipGetSymbolAddress).  Returns a hipError_t value as int.
constexpr size_t kRopeIndexScratchBytes = MROPE_ROPE_INDEX_SCRATCH_BYTES;
int rope_index_scratch(void** out);
int launch_vision_pos_ids(const VisionPosParams& p, void* stream);

// Launchers (mrope_kernels.hip).  Return a hipError_t value as int.
// nt_cap bounds the tokens per wavefront (its cos/sin LDS slice holds
// 2 * nt * half binary32 values, and a tile's byte extent must fit 31 bits).
// prec: MROPE_PRECISION_EXACT or _DTYPE, or _FP32 for bf16 (the host maps
// binary32 FP32 to DTYPE, the same arithmetic).
int launch_qk(int dtype, int vec, int cs_mode, bool norm, int prec, const QKParams& p,
              const ColTable& tab, int nt_cap, void* stream);
int launch_cos_sin(const CosSinParams& p, const ColTable& tab, void* stream);
// The pipelined q/k kernel (positions path, 16-byte chunks: vec 8 for bf16, 4
// for binary32; one wavefront per token; two row-steps of loads in flight
// while a step is finished).
int launch_qk_pipe(int dtype, int vec, bool norm, int prec, const QKParams& p,
                   const ColTable& tab, void* stream);
// The flat q/k kernel (mrope_flat.hip): positions path without RMSNorm, one
// token per wavefront, the token's blocks read as consecutive chunks.
int launch_flat(int dtype, int vec, int prec, const QKParams& p, const ColTable& tab,
                void* stream);
// The staged kernel with G tokens per block (G in 1, 2, 4, 8, 16), and the
// LDS bytes one block of it takes.
int launch_stage(int dtype, int prec, int G, const QKParams& p, const ColTable& tab,
                 void* stream);
int stage_lds_bytes(int dtype, int G, const QKParams& p);
// 16-byte chunks of the copied tensor (v) a staged block holds in registers.
int stage_max_v_chunks();
// cos/sin cache by position: cache[(p * n_freq + i) * 2 + {0, 1}] = (cos, sin)
// of fl32(float(p) * tab.inv[i]) for p < rows, i < n_freq.
int launch_cos_sin_cache(const ColTable& tab, int n_freq, int rows, float* cache, void* stream);
// The group kernel (mrope_planes.hip): positions path without RMSNorm, full
// rotary, p.nt tokens per block; a tensor's chunks of a group (heads * nt *
// D / V) at most planes_max_chunks_per_tensor(), nt * half at most
// planes_max_cos_sin(), half a multiple of V / 2.
int launch_planes(int dtype, int prec, const QKParams& p, const ColTable& tab, void* stream);
int planes_max_chunks_per_tensor();
int planes_max_cos_sin();
// Plain streaming copy of `bytes` (a multiple of 16, 16-byte aligned buffers)
// (mrope_copy.hip).
int launch_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

}  // namespace mrope
