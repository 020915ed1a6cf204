// Device-side building blocks shared by the attention kernels of libsta
// (forward in sta_attention.hip, backward in sta_backward.hip): kernel
// parameters, work-item decoding and the window walk, raster-order
// addressing, the LDS layout of K/V-like chunks and their direct-to-LDS loads.
//
// Included only by HIP translation units; everything sits in an anonymous
// namespace, so each includer gets its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "sta_kernels.h"

namespace sta {
namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kXcds = 8;  // MI355X dispatches workgroups round-robin over 8 XCDs

// Parameters shared by both kernels.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;       // optional: log-sum-exp of every query row (natural log)
  int S;            // tokens per (batch, head)
  int heads;
  int n_tasks;      // work items
  int per_xcd;      // workgroups each XCD runs (the grid is kXcds * per_xcd)
  int group;        // logical tasks an XCD takes in a row before the next XCD's turn
  int row_blocks;   // work items per query unit
  int n_units;      // query units per (batch, head): tiles, or 1 if dense
  int unit_rows;    // rows per query unit: tau, or S if dense
  float scale_log2; // scale * log2(e)
  int dense;
  int nt, nh, nw, tau;
  int H, W, ct, ch, cw;  // volume and tile, for raster-order addressing
  int T;
  int pad;               // the tile grid reaches past the volume (padded tiles)
  // Raster order, key chunks of 64 rows that each lie inside one t-plane of
  // one tile (64 divides c_h * c_w, c_w divides 64, tau a multiple of 64):
  // chunks per tile and per plane. 0 when that does not hold.
  int plane_cpt, plane_cpp;
  uint16_t omega[STA_MAX_HEADS][3];
  uint8_t head_order[STA_MAX_HEADS];  // logical head slot -> head (heaviest windows first)
};


// Maps the hardware workgroup id to a logical task so that consecutive
// logical tasks (the row blocks of one query tile, then neighbouring tiles
// that share most of their keys) run on the same XCD and share its L2.
__device__ __forceinline__ int logical_task(const AttnParams& p) {
  const int bid = blockIdx.x;
  const int x = bid % kXcds, r = bid / kXcds;
  return (r / p.group) * (kXcds * p.group) + x * p.group + r % p.group;
}

// Host side: order the work and size the grid. With equal windows on every
// head, each XCD takes one contiguous share of the tasks (group = share), so
// neighbouring tiles, which read mostly the same keys, meet in one L2. With
// unequal windows the heads are ordered by window size, heaviest first, and
// the XCDs take turns in blocks of kMixedGroup tasks: every XCD then gets the
// same mix of heavy and light work, and the light work comes last.
constexpr int kMixedGroup = 32;

// Host side: plane_cpt / plane_cpp of a sparse problem (needs tau, ch, cw).
inline void set_plane_chunks(AttnParams* p) {
  const int plane = p->ch * p->cw;
  if (!p->pad && p->tau % 64 == 0 && plane % 64 == 0 && 64 % p->cw == 0) {
    p->plane_cpt = p->tau / 64;
    p->plane_cpp = plane / 64;
  } else {
    p->plane_cpt = p->plane_cpp = 0;
  }
}

inline void plan_tasks(AttnParams* p, long long tasks, int heads, bool dense) {
  p->n_tasks = (int)tasks;
  int cost[STA_MAX_HEADS];
  bool equal = true;
  for (int h = 0; h < heads; ++h) {
    cost[h] = dense ? 1 : p->omega[h][0] * p->omega[h][1] * p->omega[h][2];
    p->head_order[h] = (uint8_t)h;
    equal = equal && cost[h] == cost[0];
  }
  const long long share = (tasks + kXcds - 1) / kXcds;
  if (equal) {
    p->group = (int)(share > 0 ? share : 1);
    p->per_xcd = p->group;
    return;
  }
  for (int i = 1; i < heads; ++i) {  // stable insertion sort, descending cost
    const uint8_t h = p->head_order[i];
    int j = i;
    while (j > 0 && cost[p->head_order[j - 1]] < cost[h]) {
      p->head_order[j] = p->head_order[j - 1];
      --j;
    }
    p->head_order[j] = h;
  }
  p->group = kMixedGroup;
  const long long blocks = (tasks + (long long)kXcds * kMixedGroup - 1) / ((long long)kXcds * kMixedGroup);
  p->per_xcd = (int)(blocks * kMixedGroup);
}

// Key runs of one work item: `runs` runs of `run_len` tokens; run r starts at
// token run_start(r).
struct KvRuns {
  int runs, run_len;
  int oh;             // omega_h (runs per t-step)
  int st, sh, sw;     // window start in tiles
  int nh, nw, tau;
  int dense;
  // Token index (tile-major order) of run r's first key.
  __device__ __forceinline__ int run_start(int r) const {
    if (dense) return 0;
    const int it = r / oh, ih = r - (r / oh) * oh;
    return (((st + it) * nh + (sh + ih)) * nw + sw) * tau;
  }
  // Raster token index of run r's first key (the run's tile-major key e sits
  // at this plus the run offset table entry e).
  __device__ __forceinline__ int run_start_raster(int r, int H, int W, int ct, int ch, int cw) const {
    const int it = r / oh, ih = r - (r / oh) * oh;
    return (((st + it) * ct) * H + (sh + ih) * ch) * W + sw * cw;
  }
};

struct Task {
  long long head_base;  // element offset of this (batch, head)
  int row0;             // first query row (token index) of the work item
  int valid_rows;       // rows of the work item inside its unit
  int local0;           // first row of the work item within its unit
  int qt, qh, qw;       // query tile coordinates (STA)
  KvRuns kv;
};

// Whether row `local` (tile-major order inside the tile) of tile (qt, qh, qw)
// is a token of the volume (false for padding positions of a partly padded
// tile).
__device__ __forceinline__ bool tile_row_real(const AttnParams& p, int qt, int qh, int qw, int local) {
  const int plane = p.ch * p.cw;
  const int lt = local / plane;
  const int rem = local - lt * plane;
  const int lh = rem / p.cw;
  const int lw = rem - lh * p.cw;
  return qt * p.ct + lt < p.T && qh * p.ch + lh < p.H && qw * p.cw + lw < p.W;
}

// Whether run r of a walk reaches past the volume (only then can its keys
// include padding positions).
__device__ __forceinline__ bool run_padded(const AttnParams& p, const KvRuns& kv, int r) {
  const int it = r / kv.oh, ih = r - (r / kv.oh) * kv.oh;
  const int tiles_w = kv.run_len / kv.tau;
  return (kv.st + it + 1) * p.ct > p.T || (kv.sh + ih + 1) * p.ch > p.H ||
         (kv.sw + tiles_w) * p.cw > p.W;
}

// Whether key e (tile-major order within the run) of run r is a token.
__device__ __forceinline__ bool run_key_real(const AttnParams& p, const KvRuns& kv, int r, int e) {
  const int it = r / kv.oh, ih = r - (r / kv.oh) * kv.oh;
  const int tw = e / p.tau;
  return tile_row_real(p, kv.st + it, kv.sh + ih, kv.sw + tw, e - tw * p.tau);
}

// Raster token index of row `local` (tile-major order inside the tile) of
// query tile (qt, qh, qw).
__device__ __forceinline__ int tile_row_raster(const AttnParams& p, int qt, int qh, int qw, int local) {
  const int plane = p.ch * p.cw;
  const int lt = local / plane;
  const int rem = local - lt * plane;
  const int lh = rem / p.cw;
  const int lw = rem - lh * p.cw;
  return ((qt * p.ct + lt) * p.H + qh * p.ch + lh) * p.W + qw * p.cw + lw;
}

// Raster offset, relative to the run's first key, of key e of a window run
// (tile-major order within the run: tile along w, then the tile's tokens).
__device__ __forceinline__ int run_offset_raster(const AttnParams& p, int e) {
  const int tw = e / p.tau;
  const int local = e - tw * p.tau;
  const int plane = p.ch * p.cw;
  const int lt = local / plane;
  const int rem = local - lt * plane;
  const int lh = rem / p.cw;
  const int lw = rem - lh * p.cw;
  return (lt * p.H + lh) * p.W + tw * p.cw + lw;
}

// Work item `task`: its (batch, head), its block of rows inside one unit, and
// the runs of the other side it walks. Forward (KEYS = false): the unit is a
// query tile and the runs cover the key tiles of its window. Backward over
// keys (KEYS = true): the unit is a key tile and the runs cover the query
// tiles whose window holds it (per axis an interval, window_inverse).
template <int ROWS, bool KEYS = false>
__device__ __forceinline__ Task decode_task(const AttnParams& p, int task, int D) {
  Task t;
  const int rb = task % p.row_blocks;
  const int unit_bh = task / p.row_blocks;
  const int unit = unit_bh % p.n_units;
  const int bh = unit_bh / p.n_units;
  const int h = p.head_order[bh % p.heads];
  t.head_base = ((long long)(bh / p.heads) * p.heads + h) * p.S * D;
  const int unit_row0 = unit * p.unit_rows;
  t.row0 = unit_row0 + rb * ROWS;
  t.local0 = rb * ROWS;
  t.valid_rows = min(ROWS, p.unit_rows - rb * ROWS);
  t.qt = t.qh = t.qw = 0;
  KvRuns& kv = t.kv;
  kv.dense = p.dense;
  kv.nh = p.nh; kv.nw = p.nw; kv.tau = p.tau;
  if (p.dense) {
    kv.runs = 1; kv.run_len = p.S; kv.oh = 1; kv.st = kv.sh = kv.sw = 0;
  } else {
    const int ot = p.omega[h][0], oh = p.omega[h][1], ow = p.omega[h][2];
    const int qw = unit % p.nw;
    const int qh = (unit / p.nw) % p.nh;
    const int qt = unit / (p.nw * p.nh);
    t.qt = qt; t.qh = qh; t.qw = qw;
    if (KEYS) {
      int lo_t, hi_t, lo_h, hi_h, lo_w, hi_w;
      window_inverse(qt, p.nt, ot, &lo_t, &hi_t);
      window_inverse(qh, p.nh, oh, &lo_h, &hi_h);
      window_inverse(qw, p.nw, ow, &lo_w, &hi_w);
      kv.st = lo_t; kv.sh = lo_h; kv.sw = lo_w;
      kv.oh = hi_h - lo_h + 1;
      kv.runs = (hi_t - lo_t + 1) * kv.oh;
      kv.run_len = (hi_w - lo_w + 1) * p.tau;
    } else {
      kv.st = window_start(qt, p.nt, ot);
      kv.sh = window_start(qh, p.nh, oh);
      kv.sw = window_start(qw, p.nw, ow);
      kv.oh = oh;
      kv.runs = ot * oh;
      kv.run_len = ow * p.tau;
    }
  }
  return t;
}

// Max / sum of x over the four lanes l, l^16, l^32, l^48 (the lanes that
// hold one query row in the MFMA output layouts). A permlane swap of x with
// itself yields, in its two results, x of this lane and of its partner lane
// (l^16 for the 16-lane swap, l^32 for the 32-lane swap), in some order.
__device__ __forceinline__ float pair16(float x, bool is_max) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return is_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float pair32(float x, bool is_max) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return is_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float row_max4(float x) { return pair32(pair16(x, true), true); }
__device__ __forceinline__ float row_sum4(float x) { return pair32(pair16(x, false), false); }
__device__ __forceinline__ float wave_xor_sum(float x, int mask) {
  return x + __shfl_xor(x, mask, 64);
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------

// QK8: Q and K are fp8 (OCP e4m3), one byte an element; S^T = K Q^T then
// takes one v_mfma_f32_16x16x128_f8f6f4 per 128 dimensions, and V, P and O
// stay bf16. KGeom is the K buffer's geometry (its rows are half as long).
template <int D, int WAVES, int RB, int BN, bool QK8 = false>
struct Bf16Cfg {
  static constexpr int kD = D;
  static constexpr int kBN = BN;
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kRowsWave = 16 * RB;
  static constexpr int kRows = WAVES * kRowsWave;
  static constexpr bool kQK8 = QK8;
  static constexpr int kDK = QK8 ? D / 128 : D / 32;   // k-steps of S^T = K Q^T
  static constexpr int kKOffs = QK8 ? 2 * kDK : kDK;    // 16-byte K reads per score tile
  using QFrag = typename std::conditional<QK8, i32x8, bf16x8>::type;
  static constexpr int kDB = D / 16;            // 16-row blocks of O^T
  static constexpr int kKT = BN / 16;           // 16-key score tiles per chunk
  static constexpr int kKP = BN / 32;           // 32-key steps of O^T += V^T P^T
  static constexpr int kRowBytes = D * 2;       // one key row of K or V
  static constexpr int kCPR = kRowBytes / 16;   // 16-byte chunks per row
  static constexpr int kChunkBytes = BN * kRowBytes;       // K (or V) of one chunk
  static constexpr int kBlocks = kChunkBytes / 1024;       // 1 KB LDS-DMA blocks per chunk
  static constexpr int kRowsPerBlock = 1024 / kRowBytes;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(!QK8 || D % 128 == 0, "fp8 scores need whole 128-dim steps");
  struct KGeom {
    static constexpr int kRowBytes = QK8 ? D : 2 * D;
    static constexpr int kCPR = kRowBytes / 16;
    static constexpr int kChunkBytes = BN * kRowBytes;
    static constexpr int kBlocks = kChunkBytes / 1024;
    static constexpr int kRowsPerBlock = 1024 / kRowBytes;
  };
};

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// LDS DMA of BYTES (4 or 16) per lane: base + voff (bytes, this lane's) into
// LDS at dst + BYTES * lane. base and dst are wave-uniform; callers pass the
// base row through readfirstlane so that the compiler knows it (else it loops
// over the lanes to build the resource). The load goes through a buffer
// resource based at the chunk, so the per-lane offsets stay small (below
// 2 GB, which the host checks) whatever the tensor size. The buffer form, not
// the global one: with a global LDS-DMA load in a loop the compiler can no
// longer count LDS reads in order and waits for all of them at every use,
// which defeats issuing operand reads ahead.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void* base, int voff, void* dst) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
  static_assert(BYTES == 4 || BYTES == 16, "LDS DMA of 4 or 16 bytes per lane");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, voff, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 4, voff, 0, 0, 0);
}

// Physical byte offset of 16-byte chunk `c` of key row `row` in a K/V buffer.
// Chunks are XOR-swizzled by the row (slot c ^ (row % CPR)) so that the
// operand fetches of the MFMA loops are not serialised on a few LDS banks:
// every row is a whole number of bank rows, so without the swizzle all rows
// of a fetch would hit the same banks. Measured on gfx950 with 256-byte rows:
// the row-wise fetch (one 16-byte chunk of 16 consecutive rows per lane
// group, ds_read_b128) runs at 215 B/clk per CU with this swizzle against 153
// with c ^ rotl4(row % 16), and the transposing fetch (ds_read_b64_tr_b16)
// runs at the same rate under either.
template <int CPR>
__device__ __forceinline__ int swz(int row, int c) {
  return row * (CPR * 16) + ((c ^ (row % CPR)) << 4);
}

// Issue this wave's share of the direct-to-LDS loads of one K (or V) chunk:
// key rows kv_row0 + key_base .. + BN - 1 of the head (rows past `nvalid`
// repeat the last valid row; their scores are masked). Each instruction fills
// one 1 KB block; WAVES wavefronts share the chunk. Keys whose bit in `real`
// is clear are padding positions: they load row kv_row0 instead, which the
// caller points at a token (the run's first key in raster order, the first
// row of the chunk's first tile in tile-major order), so that whatever a
// caller keeps in the padding rows of a tile-major tensor never reaches the
// products (a masked key still multiplies its V row by P = 0).
template <class C, int WAVES>
__device__ __forceinline__ void load_rows(const void* src, int kv_row0, int nvalid, char* buf,
                                          int wave, int lane, const int* rtab = nullptr,
                                          unsigned long long real = ~0ull, int key_base = 0) {
  constexpr int kIter = (C::kBlocks + WAVES - 1) / WAVES;
#pragma unroll
  for (int b = 0; b < kIter; ++b) {
    const int blk = wave + WAVES * b;
    if (kIter * WAVES != C::kBlocks && blk >= C::kBlocks) break;  // wave-uniform
    const int row = blk * C::kRowsPerBlock + lane / C::kCPR;
    const int pos = lane % C::kCPR;                      // slot this lane fills
    const int c = pos ^ ((swz<C::kCPR>(row, 0) >> 4) & (C::kCPR - 1));  // chunk it holds
    // Tile-major order: the chunk's keys are consecutive token rows from
    // kv_row0. Raster order: kv_row0 is the run's first raster token and
    // rtab (already offset to the chunk) gives each key's raster offset.
    const int key = min(row, nvalid - 1);
    int rel = rtab ? rtab[key] : key_base + key;
    if (!((real >> key) & 1ull)) rel = 0;
    lds_dma<16>(static_cast<const char*>(src) +
                    (long long)__builtin_amdgcn_readfirstlane(kv_row0) * C::kRowBytes,
                rel * C::kRowBytes + c * 16, buf + blk * 1024);
  }
}

// The same loads when every key of the chunk lies in one t-plane of one tile
// (plane_cpt > 0): the raster row of key `row` of the chunk is
// chunk_row0 + lane_row[b], with lane_row the row's offset inside its plane
// ((row / c_w) * W + row % c_w), computed once per lane.
template <class C, int WAVES>
__device__ __forceinline__ int plane_iters() { return (C::kBlocks + WAVES - 1) / WAVES; }

template <class C, int WAVES>
__device__ __forceinline__ void plane_lane_rows(const AttnParams& p, int wave, int lane,
                                                int (&lane_row)[(C::kBlocks + WAVES - 1) / WAVES]) {
  constexpr int kIter = (C::kBlocks + WAVES - 1) / WAVES;
#pragma unroll
  for (int b = 0; b < kIter; ++b) {
    const int row = (wave + WAVES * b) * C::kRowsPerBlock + lane / C::kCPR;
    lane_row[b] = (row / p.cw) * p.W + row % p.cw;
  }
}

template <class C, int WAVES>
__device__ __forceinline__ void load_rows_plane(const void* src, int chunk_row0,
                                                const int (&lane_row)[(C::kBlocks + WAVES - 1) / WAVES],
                                                char* buf, int wave, int lane) {
  constexpr int kIter = (C::kBlocks + WAVES - 1) / WAVES;
#pragma unroll
  for (int b = 0; b < kIter; ++b) {
    const int blk = wave + WAVES * b;
    if (kIter * WAVES != C::kBlocks && blk >= C::kBlocks) break;  // wave-uniform
    const int row = blk * C::kRowsPerBlock + lane / C::kCPR;
    const int pos = lane % C::kCPR;
    const int c = pos ^ ((swz<C::kCPR>(row, 0) >> 4) & (C::kCPR - 1));
    lds_dma<16>(static_cast<const char*>(src) +
                    (long long)__builtin_amdgcn_readfirstlane(chunk_row0) * C::kRowBytes,
                lane_row[b] * C::kRowBytes + c * 16, buf + blk * 1024);
  }
}

__device__ __forceinline__ void wait_vm_all() {
  // vmcnt(0); expcnt and lgkmcnt left at their maxima (not waited on).
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Rare branches (a ragged last chunk, a growing row max) hold code the
// compiler would otherwise turn into unconditional selects and multiplies on
// every chunk; an empty volatile asm statement keeps them real branches.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Token index (in the tensor's own order) of each of this lane's query rows,
// and whether the row exists (work items may be ragged).
template <class C, int RB>
struct RowMap {
  int tok[RB];
  bool ok[RB];
};

template <class C, int RB, bool RASTER>
__device__ __forceinline__ RowMap<C, RB> map_rows(const AttnParams& p, const Task& t, int wave,
                                                  int l16) {
  RowMap<C, RB> rm;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wave * C::kRowsWave + 16 * rb + l16;
    rm.ok[rb] = r < t.valid_rows &&
                (!p.pad || tile_row_real(p, t.qt, t.qh, t.qw, t.local0 + r));
    // rows that do not exist read the unit's first row (a token of every tile,
    // also of a partly padded one) and are never stored
    const int local = rm.ok[rb] ? t.local0 + r : 0;
    rm.tok[rb] = RASTER ? tile_row_raster(p, t.qt, t.qh, t.qw, local) : t.row0 - t.local0 + local;
  }
  return rm;
}

// Walks the key chunks of a work item: chunk `it` covers keys
// row0(it) .. + BN of the head, of which nvalid(it) are inside the run.
struct ChunkWalk {
  int chunks_per_run, n_chunks, run_len, bn;
  KvRuns kv;
  bool dense;
  __device__ __forceinline__ void at(int it, int* row0, int* nvalid) const {
    const int run = it / chunks_per_run;
    const int c0 = (it - run * chunks_per_run) * bn;
    *row0 = (dense ? 0 : kv.run_start(run)) + c0;
    *nvalid = min(bn, run_len - c0);
  }
  // Raster order, plane chunks: the raster token of the chunk's first key
  // (the chunk is one 64-row piece of one t-plane of one tile).
  __device__ __forceinline__ int at_plane(const AttnParams& p, int it) const {
    const int run = it / chunks_per_run;
    const int j = it - run * chunks_per_run;
    const int tw = j / p.plane_cpt;
    const int pp = j - tw * p.plane_cpt;
    const int lt = pp / p.plane_cpp;
    const int sub = pp - lt * p.plane_cpp;
    return kv.run_start_raster(run, p.H, p.W, p.ct, p.ch, p.cw) +
           (lt * p.H + sub * (64 / p.cw)) * p.W + tw * p.cw;
  }
  // Tile-major order on a padded grid: the first row of the tile the chunk
  // starts in (a token: every tile starts inside the volume), the chunk's
  // first key relative to it, and the number of valid keys.
  __device__ __forceinline__ void at_tile(int it, int tau, int* tile_row0, int* key_base,
                                          int* nvalid) const {
    const int run = it / chunks_per_run;
    const int c0 = (it - run * chunks_per_run) * bn;
    *key_base = c0 % tau;
    *tile_row0 = (dense ? 0 : kv.run_start(run)) + c0 - *key_base;
    *nvalid = min(bn, run_len - c0);
  }
  // Raster order: the run's first raster token, the chunk's first key within
  // the run, and the number of valid keys.
  __device__ __forceinline__ void at_raster(const AttnParams& p, int it, int* base, int* c0,
                                            int* nvalid) const {
    const int run = it / chunks_per_run;
    *c0 = (it - run * chunks_per_run) * bn;
    *base = kv.run_start_raster(run, p.H, p.W, p.ct, p.ch, p.cw);
    *nvalid = min(bn, run_len - *c0);
  }
};

// Bit k set iff key k (0..63) of chunk `it` is a token of the volume: all
// ones unless the problem is padded (PAD, a kernel variant of its own so that
// unpadded launches carry no masking code) and the chunk's run reaches past
// the volume. One key per lane (64-key chunks), then a wave ballot.
template <bool PAD>
__device__ __forceinline__ unsigned long long chunk_real_keys(const AttnParams& p, const ChunkWalk& w,
                                                               int it, int lane) {
  if (!PAD) return ~0ull;
  const int run = it / w.chunks_per_run;
  if (!run_padded(p, w.kv, run)) return ~0ull;
  const int e = (it - run * w.chunks_per_run) * w.bn + lane;
  const bool real = e < w.run_len && run_key_real(p, w.kv, run, e);
  return __ballot(real);
}

template <int BN, bool DENSE>
__device__ __forceinline__ ChunkWalk make_walk(const Task& t, int S) {
  ChunkWalk cw;
  cw.kv = t.kv;
  cw.dense = DENSE;
  cw.run_len = DENSE ? S : t.kv.run_len;
  cw.bn = BN;
  cw.chunks_per_run = (cw.run_len + BN - 1) / BN;
  cw.n_chunks = (DENSE ? 1 : t.kv.runs) * cw.chunks_per_run;
  return cw;
}

}  // namespace
}  // namespace sta
