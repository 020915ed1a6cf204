// Attention kernels of libsta (gfx950): Sliding Tile Attention forward and
// the dense comparator.
//
// Work decomposition. A work item is a block of query rows that lies inside
// one query tile (STA) or one slice of the sequence (dense). Every row of a
// tile attends to the same keys: the tiles of the tile's window. In tile-major
// memory the window is omega_t * omega_h runs, each run omega_w consecutive
// tiles = omega_w * tau consecutive tokens. The kernel walks those runs in
// chunks of BN keys, so no block is ever masked except for a ragged last chunk
// of a run whose length is not a multiple of BN.
//
// bf16 kernel. Each wavefront owns RB blocks of 16 query rows. It computes
// S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (K from LDS as the A operand, the
// wave's Q rows held in registers as the B operand), so every lane ends up
// holding scores of a single query row. The online softmax (base 2, scale
// folded into one multiply) runs on those registers; the probabilities are
// rounded to bf16 and used directly as the B operand of O^T = V^T P^T, whose
// A operand is V transposed in LDS. The accumulator O^T again keeps one query
// row per lane, so the softmax rescale is a per-lane scalar.
//
// f32 kernel. One thread per query row, K/V chunks staged in LDS, plain fp32
// FMA arithmetic; it serves float32 problems.
#include <hip/hip_runtime.h>

#include "sta_kernels.h"

namespace sta {
namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;  // MI355X dispatches workgroups round-robin over 8 XCDs

// Parameters shared by both kernels.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int S;            // tokens per (batch, head)
  int heads;
  int n_tasks;      // work items
  int per_xcd;      // ceil(n_tasks / kXcds)
  int row_blocks;   // work items per query unit
  int n_units;      // query units per (batch, head): tiles, or 1 if dense
  int unit_rows;    // rows per query unit: tau, or S if dense
  float scale_log2; // scale * log2(e)
  int dense;
  int nt, nh, nw, tau;
  int H, W, ct, ch, cw;  // volume and tile, for raster-order addressing
  uint16_t omega[STA_MAX_HEADS][3];
};


// Maps the hardware workgroup id to a logical task so that consecutive
// logical tasks (the row blocks of one query tile, then neighbouring tiles
// that share most of their keys) run on the same XCD and share its L2.
__device__ __forceinline__ int logical_task(const AttnParams& p) {
  const int bid = blockIdx.x;
  return (bid % kXcds) * p.per_xcd + bid / kXcds;
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

template <int ROWS>
__device__ __forceinline__ Task decode_task(const AttnParams& p, int task, int D) {
  Task t;
  const int rb = task % p.row_blocks;
  const int unit_bh = task / p.row_blocks;
  const int unit = unit_bh % p.n_units;
  const int bh = unit_bh / p.n_units;
  const int h = bh % p.heads;
  t.head_base = (long long)bh * p.S * D;
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
    kv.st = window_start(qt, p.nt, ot);
    kv.sh = window_start(qh, p.nh, oh);
    kv.sw = window_start(qw, p.nw, ow);
    kv.oh = oh;
    kv.runs = ot * oh;
    kv.run_len = ow * p.tau;
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

template <int D, int WAVES, int RB, int BN>
struct Bf16Cfg {
  static constexpr int kD = D;
  static constexpr int kBN = BN;
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kRowsWave = 16 * RB;
  static constexpr int kRows = WAVES * kRowsWave;
  static constexpr int kDK = D / 32;            // k-steps of S^T = K Q^T
  static constexpr int kDB = D / 16;            // 16-row blocks of O^T
  static constexpr int kKT = BN / 16;           // 16-key score tiles per chunk
  static constexpr int kKP = BN / 32;           // 32-key steps of O^T += V^T P^T
  static constexpr int kRowBytes = D * 2;       // one key row of K or V
  static constexpr int kCPR = kRowBytes / 16;   // 16-byte chunks per row
  static constexpr int kChunkBytes = BN * kRowBytes;       // K (or V) of one chunk
  static constexpr int kBlocks = kChunkBytes / 1024;       // 1 KB LDS-DMA blocks per chunk
  static constexpr int kRowsPerBlock = 1024 / kRowBytes;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
};

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Physical byte offset of 16-byte chunk `c` of key row `row` in a K/V buffer.
// Chunks are XOR-swizzled by the row so that the operand fetches of the MFMA
// loops hit distinct LDS banks: with 256-byte rows every row starts at bank 0
// and the chunk slot is c ^ rotl4(row % 16). The K fetch reads one chunk of
// 16 consecutive rows (rotl4 is a bijection on 0..15); the transposing V
// fetch reads chunks 2m and 2m+1 of 8 consecutive rows, which rotl4 also
// spreads over 16 distinct slots. With 128-byte rows the slot is c ^ (row % 8).
template <int CPR>
__device__ __forceinline__ int swz(int row, int c) {
  int key;
  if (CPR == 16) {
    const int r = row & 15;
    key = ((r << 1) | (r >> 3)) & 15;
  } else {
    key = row % CPR;
  }
  return row * (CPR * 16) + ((c ^ key) << 4);
}

// Issue this wave's share of the direct-to-LDS loads of one K (or V) chunk:
// key rows kv_row0 .. kv_row0 + BN - 1 of the head (rows past `nvalid` repeat
// the last valid row; their scores are masked). Each instruction fills one
// 1 KB block; WAVES wavefronts share the chunk.
template <class C, int WAVES>
__device__ __forceinline__ void load_rows(const bf16_t* src, int kv_row0, int nvalid, char* buf,
                                          int wave, int lane, const int* rtab = nullptr) {
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
    const int src_row = rtab ? kv_row0 + rtab[key] : kv_row0 + key;
    const long long off = (long long)src_row * (C::kRowBytes / 2) + c * 8;
    __builtin_amdgcn_global_load_lds(src + off, (lds_void*)(buf + blk * 1024), 16, 0, 0);
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

// Per-wave state of the flash loop: Q fragments, O^T accumulators, running
// max m (log2 units) and partial row sums, the current scores and the bf16
// probabilities, and the lane's byte offsets into a K/V buffer.
template <class C, int RB>
struct WaveState {
  bf16x8 qf[RB][C::kDK];
  f32x4 o[RB][C::kDB];
  float m[RB], lsum[RB];
  f32x4 s[RB][C::kKT];
  bf16x8 pf[RB][C::kKP];
  // K operand: row 16*kt + l16, chunk 4*dk + g; the swizzled offset is
  // koff[dk] + 16*kt*row_bytes because the row's low 4 bits are l16.
  int koff[C::kDK];
  // V operand (transposing read): row 32*kp + 4g + l16/4 (+16 for the upper
  // half), element column 16*db + 4*(l16 % 4); offset voff[db] + rows*row_bytes.
  int voff[C::kDB];
};

template <class C, int RB>
__device__ __forceinline__ void lane_offsets(WaveState<C, RB>& w, int l16, int g) {
#pragma unroll
  for (int dk = 0; dk < C::kDK; ++dk) w.koff[dk] = swz<C::kCPR>(l16, 4 * dk + g);
  const int s4 = l16 >> 2, sq = l16 & 3;
  const int vrow = 4 * g + s4;  // row within its 16-row group (< 16)
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
    const int col = 16 * db + 4 * sq;
    w.voff[db] = swz<C::kCPR>(vrow, col >> 3) + (col & 7) * 2;
  }
}

// Scores S^T[key][row] = K Q^T for one chunk; lane (l16, g) ends up with keys
// 16*kt + 4g + r of query row l16 of each 16-row block.
template <class C, int RB>
__device__ __forceinline__ void qk_into(WaveState<C, RB>& w, f32x4 (&sc)[RB][C::kKT],
                                        const char* kbuf, int l16, int g) {
#pragma unroll
  for (int kt = 0; kt < C::kKT; ++kt) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sc[rb][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dk = 0; dk < C::kDK; ++dk) {
      const bf16x8 kf =
          *reinterpret_cast<const bf16x8*>(kbuf + w.koff[dk] + 16 * kt * C::kRowBytes);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        sc[rb][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, w.qf[rb][dk], sc[rb][kt], 0, 0, 0);
    }
  }
}

template <class C, int RB>
__device__ __forceinline__ void qk_chunk(WaveState<C, RB>& w, const char* kbuf, int l16, int g) {
  qk_into<C, RB>(w, w.s, kbuf, l16, g);
}

template <class C, int RB>
__device__ __forceinline__ void softmax_max(WaveState<C, RB>& w, f32x4 (&sc)[RB][C::kKT],
                                            int nvalid, float scale_log2, int g) {
  if (nvalid < C::kBN) {
    keep_branch();
#pragma unroll
    for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * kt + 4 * g + r >= nvalid)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) sc[rb][kt][r] = -INFINITY;
  }
  float mx[RB];
  bool grow = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float a = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::kKT; ++kt)
      a = fmaxf(a, fmaxf(fmaxf(sc[rb][kt][0], sc[rb][kt][1]), fmaxf(sc[rb][kt][2], sc[rb][kt][3])));
    mx[rb] = row_max4(a) * scale_log2;
    grow |= mx[rb] > w.m[rb] + 8.0f;
  }
  if (__any(grow)) {
    keep_branch();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float m_new = fmaxf(w.m[rb], mx[rb]);
      const float alpha = __builtin_amdgcn_exp2f(w.m[rb] - m_new);
      w.m[rb] = m_new;
      w.lsum[rb] *= alpha;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) w.o[rb][db] *= alpha;
    }
  }
}

template <class C, int RB>
__device__ __forceinline__ void softmax_exp(WaveState<C, RB>& w, f32x4 (&sc)[RB][C::kKT],
                                            float scale_log2) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sc[rb][kt][r] = __builtin_amdgcn_exp2f(fmaf(sc[rb][kt][r], scale_log2, -w.m[rb]));
    // The row sum adds the bf16-rounded probabilities, the same values that
    // multiply V, two per dot instruction.
    float ls = w.lsum[rb];
    const bf16x2 ones = {static_cast<bf16_t>(1.0f), static_cast<bf16_t>(1.0f)};
#pragma unroll
    for (int kp = 0; kp < C::kKP; ++kp) {
      bf16x8 x;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = static_cast<bf16_t>(sc[rb][2 * kp][r]);
        x[4 + r] = static_cast<bf16_t>(sc[rb][2 * kp + 1][r]);
      }
      w.pf[rb][kp] = x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {x[2 * e], x[2 * e + 1]};
        ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls, false);
      }
    }
    w.lsum[rb] = ls;
  }
}

// Online softmax (base 2) of one chunk's scores into bf16 probabilities. The
// reference max m only moves when a row's chunk max exceeds it by more than 8
// (then O and the row sum are rescaled); in between, probabilities stay below
// 2^8, which fp32 sums and bf16 P hold as well as values below 1.
template <class C, int RB>
__device__ __forceinline__ void softmax_chunk(WaveState<C, RB>& w, int nvalid, float scale_log2,
                                              int g) {
  softmax_max<C, RB>(w, w.s, nvalid, scale_log2, g);
  softmax_exp<C, RB>(w, w.s, scale_log2);
}

// O^T[d][row] += V^T[d][key] P^T[key][row] for one chunk. Slot j of lane group
// g maps to key 32*kp + 4g + j (j < 4) or 32*kp + 16 + 4g + (j - 4). The
// transposing LDS read gives lane i of a 16-lane group element (i % 4) of the
// 4-element piece addressed by lane 4r + i/4, for r = 0..3: lane s of group g
// addresses key 32*kp + 4g + s/4, columns 16*db + 4*(s%4) .. +4, so lane i
// receives V[32*kp + 4g + r][16*db + i], r = 0..3.
template <class C, int RB>
__device__ __forceinline__ void pv_chunk(WaveState<C, RB>& w, const char* vbuf, int l16, int g) {
#pragma unroll
  for (int kp = 0; kp < C::kKP; ++kp) {
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) {
      const char* lo_addr = vbuf + w.voff[db] + 32 * kp * C::kRowBytes;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(lo_addr));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(lo_addr + 16 * C::kRowBytes));
      const i16x4 both[2] = {lo, hi};
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(both);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        w.o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, w.pf[rb][kp], w.o[rb][db], 0, 0, 0);
    }
  }
}

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
    rm.ok[rb] = r < t.valid_rows;
    const int rr = rm.ok[rb] ? r : 0;
    rm.tok[rb] = RASTER ? tile_row_raster(p, t.qt, t.qh, t.qw, t.local0 + rr) : t.row0 + rr;
  }
  return rm;
}

template <class C, int RB>
__device__ __forceinline__ void load_q_init(WaveState<C, RB>& w, const bf16_t* qg,
                                            const RowMap<C, RB>& rm, int l16, int g) {
  lane_offsets<C, RB>(w, l16, g);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bf16_t* src = qg + (long long)rm.tok[rb] * C::kD + 8 * g;
#pragma unroll
    for (int dk = 0; dk < C::kDK; ++dk) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(src + 32 * dk);
      if (!rm.ok[rb]) x = bf16x8{};
      w.qf[rb][dk] = x;
    }
    w.m[rb] = -INFINITY;
    w.lsum[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) w.o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Normalise and store: lane holds O[row l16][16*db + 4g + r].
template <class C, int RB>
__device__ __forceinline__ void store_out(WaveState<C, RB>& w, bf16_t* og, const RowMap<C, RB>& rm,
                                          int g) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float inv = 1.0f / row_sum4(w.lsum[rb]);
    if (rm.ok[rb]) {
      bf16_t* dst = og + (long long)rm.tok[rb] * C::kD + 4 * g;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = static_cast<bf16_t>(w.o[rb][db][e] * inv);
        *reinterpret_cast<bf16x4*>(dst + 16 * db) = y;
      }
    }
  }
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

// Flash loop: every wave runs QK^T, softmax and PV of a chunk in turn; the
// next chunk's K and V stream into the other LDS buffer meanwhile.
// RASTER: q, k, v, out are in raster token order (the permutation to and from
// tile-major order is folded into the addressing): query rows map through
// tile_row_raster, and every key of a window run through a table of raster
// offsets built in dynamic LDS at the start (all runs of a work item share it).
template <int D, int WAVES, int RB, int BN, bool DENSE, bool RASTER>
__global__ void __launch_bounds__(WAVES * 64, (WAVES <= 4 ? 2 : 1))
attn_bf16_kernel(const AttnParams p) {
  using C = Bf16Cfg<D, WAVES, RB, BN>;
  // K and V buffers of two chunks. They are separate objects and the loop
  // selects them statically, so the compiler can tell the chunk being read
  // apart from the one the LDS DMA is filling and does not wait for the
  // prefetch before reading.
  __shared__ __attribute__((aligned(1024))) char kb0[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char vb0[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char kb1[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char vb1[C::kChunkBytes];
  // Raster offsets of one window run (RASTER only), sized at launch.
  extern __shared__ int rtab[];

  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<C::kRows>(p, task, D);
  const bf16_t* qg = static_cast<const bf16_t*>(p.q) + t.head_base;
  const bf16_t* kg = static_cast<const bf16_t*>(p.k) + t.head_base;
  const bf16_t* vg = static_cast<const bf16_t*>(p.v) + t.head_base;
  bf16_t* og = static_cast<bf16_t*>(p.out) + t.head_base;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const ChunkWalk walk = make_walk<BN, DENSE>(t, p.S);
  if (RASTER) {
    for (int e = threadIdx.x; e < walk.run_len; e += C::kThreads) rtab[e] = run_offset_raster(p, e);
    __syncthreads();
  }
  auto dma = [&](int it, char* kdst, char* vdst) __attribute__((always_inline)) {
    if (RASTER) {
      int base, c0, nv;
      walk.at_raster(p, it, &base, &c0, &nv);
      load_rows<C, WAVES>(kg, base, nv, kdst, wave, lane, rtab + c0);
      load_rows<C, WAVES>(vg, base, nv, vdst, wave, lane, rtab + c0);
    } else {
      int row0, nv;
      walk.at(it, &row0, &nv);
      load_rows<C, WAVES>(kg, row0, nv, kdst, wave, lane);
      load_rows<C, WAVES>(vg, row0, nv, vdst, wave, lane);
    }
  };
  dma(0, kb0, vb0);
  const RowMap<C, RB> rm = map_rows<C, RB, RASTER>(p, t, wave, l16);
  WaveState<C, RB> w;
  load_q_init<C, RB>(w, qg, rm, l16, g);

  auto chunk_step = [&](const char* kcur, const char* vcur, char* knxt, char* vnxt, int it)
                        __attribute__((always_inline)) {
    int row0, nvalid;
    walk.at(it, &row0, &nvalid);
    wait_vm_all();     // this wave's loads of chunk `it` have landed in LDS
    __syncthreads();   // ... and every wave's; chunk it-1's buffers are free
    if (it + 1 < walk.n_chunks) dma(it + 1, knxt, vnxt);
    qk_chunk<C, RB>(w, kcur, l16, g);
    softmax_chunk<C, RB>(w, nvalid, p.scale_log2, g);
    pv_chunk<C, RB>(w, vcur, l16, g);
  };
  for (int it = 0; it < walk.n_chunks; it += 2) {
    chunk_step(kb0, vb0, kb1, vb1, it);
    if (it + 1 < walk.n_chunks) chunk_step(kb1, vb1, kb0, vb0, it + 1);
  }
  store_out<C, RB>(w, og, rm, g);
}

// ---------------------------------------------------------------------------
// f32 kernel
// ---------------------------------------------------------------------------

constexpr int kF32Threads = 128;
constexpr int kF32BN = 32;

template <int D, bool RASTER>
__global__ void __launch_bounds__(kF32Threads) attn_f32_kernel(const AttnParams p) {
  __shared__ float4 ks[kF32BN * D / 4];
  __shared__ float4 vs[kF32BN * D / 4];
  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<kF32Threads>(p, task, D);
  const float* qg = static_cast<const float*>(p.q) + t.head_base;
  const float4* kg = reinterpret_cast<const float4*>(static_cast<const float*>(p.k) + t.head_base);
  const float4* vg = reinterpret_cast<const float4*>(static_cast<const float*>(p.v) + t.head_base);
  float* og = static_cast<float*>(p.out) + t.head_base;

  const int tid = threadIdx.x;
  const bool row_ok = tid < t.valid_rows;
  float q[D], o[D];
  const int my_row = row_ok ? tid : 0;
  const int q_tok = RASTER ? tile_row_raster(p, t.qt, t.qh, t.qw, t.local0 + my_row) : t.row0 + my_row;
  const float* qrow = qg + (long long)q_tok * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = row_ok ? qrow[d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int run = 0; run < t.kv.runs; ++run) {
    const int kv0 = t.kv.run_start(run);
    const int kv0_raster = RASTER ? t.kv.run_start_raster(run, p.H, p.W, p.ct, p.ch, p.cw) : 0;
    for (int c0 = 0; c0 < t.kv.run_len; c0 += kF32BN) {
      const int nvalid = min(kF32BN, t.kv.run_len - c0);
      __syncthreads();
      for (int i = tid; i < kF32BN * D / 4; i += kF32Threads) {
        const int key = i / (D / 4);
        float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
        if (key < nvalid) {
          const int tok = RASTER ? kv0_raster + run_offset_raster(p, c0 + key) : kv0 + c0 + key;
          const long long off = (long long)tok * (D / 4) + (i - key * (D / 4));
          kx = kg[off];
          vx = vg[off];
        }
        ks[i] = kx;
        vs[i] = vx;
      }
      __syncthreads();
      float s[kF32BN];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kF32BN; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 kk = ks[j * (D / 4) + d4];
          acc = fmaf(q[4 * d4], kk.x, acc);
          acc = fmaf(q[4 * d4 + 1], kk.y, acc);
          acc = fmaf(q[4 * d4 + 2], kk.z, acc);
          acc = fmaf(q[4 * d4 + 3], kk.w, acc);
        }
        s[j] = j < nvalid ? acc * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
      for (int j = 0; j < kF32BN; ++j) {
        const float e = __builtin_amdgcn_exp2f(s[j] - m_new);
        l += e;
#pragma unroll
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 vv = vs[j * (D / 4) + d4];
          o[4 * d4] = fmaf(e, vv.x, o[4 * d4]);
          o[4 * d4 + 1] = fmaf(e, vv.y, o[4 * d4 + 1]);
          o[4 * d4 + 2] = fmaf(e, vv.z, o[4 * d4 + 2]);
          o[4 * d4 + 3] = fmaf(e, vv.w, o[4 * d4 + 3]);
        }
      }
    }
  }
  if (row_ok) {
    const float inv = 1.0f / l;
    float* dst = og + (long long)q_tok * D;
#pragma unroll
    for (int d = 0; d < D; ++d) dst[d] = o[d] * inv;
  }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

void fill_params(const AttnProblem& pr, int rows_per_item, AttnParams* p) {
  p->q = pr.q; p->k = pr.k; p->v = pr.v; p->out = pr.out;
  p->S = pr.g.S;
  p->heads = pr.heads;
  p->dense = pr.dense ? 1 : 0;
  p->scale_log2 = pr.scale * kLog2e;
  if (pr.dense) {
    p->n_units = 1;
    p->unit_rows = pr.g.S;
    p->nt = p->nh = p->nw = 1;
    p->tau = pr.g.S;
    p->H = p->W = p->ct = p->ch = p->cw = 1;
  } else {
    p->n_units = pr.g.n_tiles;
    p->unit_rows = pr.g.tau;
    p->nt = pr.g.nt; p->nh = pr.g.nh; p->nw = pr.g.nw;
    p->tau = pr.g.tau;
    p->H = pr.g.H; p->W = pr.g.W;
    p->ct = pr.g.ct; p->ch = pr.g.ch; p->cw = pr.g.cw;
    for (int h = 0; h < pr.heads; ++h)
      for (int a = 0; a < 3; ++a) p->omega[h][a] = pr.omega[h][a];
  }
  p->row_blocks = (p->unit_rows + rows_per_item - 1) / rows_per_item;
  const long long tasks = (long long)pr.B * pr.heads * p->n_units * p->row_blocks;
  p->n_tasks = (int)tasks;
  p->per_xcd = (int)((tasks + kXcds - 1) / kXcds);
}

// LDS for the raster offsets of the longest window run, omega_w * tau keys.
unsigned raster_table_bytes(const AttnProblem& pr) {
  int run = 0;
  for (int h = 0; h < pr.heads; ++h) run = pr.omega[h][2] * pr.g.tau > run ? pr.omega[h][2] * pr.g.tau : run;
  return (unsigned)run * sizeof(int);
}

template <int D, int WAVES, int RB, int BN>
int launch_bf16(const AttnProblem& pr, hipStream_t stream) {
  using C = Bf16Cfg<D, WAVES, RB, BN>;
  AttnParams p;
  fill_params(pr, C::kRows, &p);
  const unsigned grid = (unsigned)p.per_xcd * kXcds;
  if (pr.dense)
    hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, true, false>), dim3(grid),
                       dim3(C::kThreads), 0, stream, p);
  else if (pr.raster)
    hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, true>), dim3(grid),
                       dim3(C::kThreads), raster_table_bytes(pr), stream, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, false>), dim3(grid),
                       dim3(C::kThreads), 0, stream, p);
  return (int)hipGetLastError();
}

template <int D>
int launch_f32(const AttnProblem& pr, hipStream_t stream) {
  AttnParams p;
  fill_params(pr, kF32Threads, &p);
  const unsigned grid = (unsigned)p.per_xcd * kXcds;
  if (pr.raster && !pr.dense)
    hipLaunchKernelGGL((attn_f32_kernel<D, true>), dim3(grid), dim3(kF32Threads), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, false>), dim3(grid), dim3(kF32Threads), 0, stream, p);
  return (int)hipGetLastError();
}

// Rows per bf16 work item: a whole 384-token tile when it fits, else 64 or 128.
template <int D>
int dispatch_bf16(const AttnProblem& pr, hipStream_t stream) {
  const int unit_rows = pr.dense ? pr.g.S : pr.g.tau;
#ifndef STA_CFG_WAVES
#define STA_CFG_WAVES 8
#endif
#ifndef STA_CFG_RB
#define STA_CFG_RB 3
#endif
#ifndef STA_CFG_BN
#define STA_CFG_BN 64
#endif
  constexpr int kBigRows = STA_CFG_WAVES * 16 * STA_CFG_RB;
  if (unit_rows % kBigRows == 0) return launch_bf16<D, STA_CFG_WAVES, STA_CFG_RB, STA_CFG_BN>(pr, stream);
  if (unit_rows <= 64) return launch_bf16<D, 4, 1, 64>(pr, stream);
  return launch_bf16<D, 4, 2, 64>(pr, stream);
}

}  // namespace

int launch_attention(const AttnProblem& pr, void* stream_ptr) {
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const long long units = pr.dense ? 1 : pr.g.n_tiles;
  const long long tasks_upper = (long long)pr.B * pr.heads * units * (pr.dense ? pr.g.S : pr.g.tau);
  if (tasks_upper > (1LL << 31) - 1) return (int)hipErrorInvalidValue;
  if (pr.dtype == STA_BF16) {
    if (pr.head_dim == 128) return dispatch_bf16<128>(pr, stream);
    if (pr.head_dim == 64) return dispatch_bf16<64>(pr, stream);
  } else if (pr.dtype == STA_F32) {
    if (pr.head_dim == 128) return launch_f32<128>(pr, stream);
    if (pr.head_dim == 64) return launch_f32<64>(pr, stream);
  }
  return STA_ERR_UNSUPPORTED;
}

}  // namespace sta
