// Work plan of the attention kernels of libsta: kernel parameters, the
// order in which work items are handed to the XCDs, and the integer
// decoding of a work item into its rows and the runs of keys (or queries) it
// walks. Host and device code share these definitions, so the host-side
// bounds model (tests/host) checks the very index arithmetic the kernels run.
//
// No HIP intrinsics here; everything sits in an anonymous namespace, so each
// includer gets its own copy.
#pragma once

#include <stdint.h>

#include "sta_geometry.h"
#include "sta_kernels.h"

namespace sta {
namespace {

STA_HD int imin(int a, int b) { return a < b ? a : b; }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kXcds = 8;  // MI355X dispatches workgroups round-robin over 8 XCDs

// Parameters shared by both kernels.
// 64-key chunks per tile up to which padded grids use precomputed token masks
// (tau <= 1024).
constexpr int kMaxPadChunks = 16;

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
  // Tail launch (0 otherwise): each workgroup runs one of tail_split row
  // blocks of a work item of an XCD's last round, which starts at round
  // tail_r0 of the XCD (see plan_tail_split).
  int tail_split;
  int tail_r0;
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
  // Padded grids with tau a multiple of 64 (each 64-key chunk inside one
  // tile): bit k of pad_mask[a][c] says whether key 64c + k of a tile lies
  // inside the extent of the tiles the volume's end cuts along axis a (the
  // last tile along t, h or w). A chunk's token mask is the AND of the masks
  // of the axes along which its key tile is cut. pad_cpt = tau / 64 then,
  // else 0.
  int pad_cpt;
  unsigned long long pad_mask[3][kMaxPadChunks];
  uint16_t omega[STA_MAX_HEADS][3];
  uint8_t head_order[STA_MAX_HEADS];  // logical head slot -> head (heaviest windows first)
  // Window recall in one pass (see AttnProblem); cand_chunks: entries of the
  // per-chunk candidate table in dynamic LDS (the walk's chunk count).
  int n_cand;
  int cand_chunks;
  float* lse_cand;
  long long cand_stride;
  uint16_t cand_omega[kMaxRecallCand][3];
};

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

// Host side: pad_cpt / pad_mask of a sparse problem (needs the volume, the
// tile and the tile grid).
inline void set_pad_masks(AttnParams* p) {
  p->pad_cpt = 0;
  if (!p->pad || p->tau % 64 != 0 || p->tau / 64 > kMaxPadChunks) return;
  const int ext[3] = {p->T - (p->nt - 1) * p->ct, p->H - (p->nh - 1) * p->ch,
                      p->W - (p->nw - 1) * p->cw};
  const int plane = p->ch * p->cw;
  for (int c = 0; c < p->tau / 64; ++c) {
    unsigned long long m[3] = {0ull, 0ull, 0ull};
    for (int k = 0; k < 64; ++k) {
      const int local = 64 * c + k;
      const int at[3] = {local / plane, (local % plane) / p->cw, local % p->cw};
      for (int a = 0; a < 3; ++a)
        if (at[a] < ext[a]) m[a] |= 1ull << k;
    }
    for (int a = 0; a < 3; ++a) p->pad_mask[a][c] = m[a];
  }
  p->pad_cpt = p->tau / 64;
}

inline void plan_tasks(AttnParams* p, long long tasks, int heads, bool dense) {
  p->n_tasks = (int)tasks;
  p->tail_split = p->tail_r0 = 0;
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
  STA_HD int run_start(int r) const {
    if (dense) return 0;
    const int it = r / oh, ih = r - (r / oh) * oh;
    return (((st + it) * nh + (sh + ih)) * nw + sw) * tau;
  }
  // Raster token index of run r's first key (the run's tile-major key e sits
  // at this plus the run offset table entry e).
  STA_HD int run_start_raster(int r, int H, int W, int ct, int ch, int cw) const {
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
STA_HD bool tile_row_real(const AttnParams& p, int qt, int qh, int qw, int local) {
  const int plane = p.ch * p.cw;
  const int lt = local / plane;
  const int rem = local - lt * plane;
  const int lh = rem / p.cw;
  const int lw = rem - lh * p.cw;
  return qt * p.ct + lt < p.T && qh * p.ch + lh < p.H && qw * p.cw + lw < p.W;
}

// Whether run r of a walk reaches past the volume (only then can its keys
// include padding positions).
STA_HD bool run_padded(const AttnParams& p, const KvRuns& kv, int r) {
  const int it = r / kv.oh, ih = r - (r / kv.oh) * kv.oh;
  const int tiles_w = kv.run_len / kv.tau;
  return (kv.st + it + 1) * p.ct > p.T || (kv.sh + ih + 1) * p.ch > p.H ||
         (kv.sw + tiles_w) * p.cw > p.W;
}

// Whether key e (tile-major order within the run) of run r is a token.
STA_HD bool run_key_real(const AttnParams& p, const KvRuns& kv, int r, int e) {
  const int it = r / kv.oh, ih = r - (r / kv.oh) * kv.oh;
  const int tw = e / p.tau;
  return tile_row_real(p, kv.st + it, kv.sh + ih, kv.sw + tw, e - tw * p.tau);
}

// Token mask of 64-key chunk `it` of walk w from the tables (pad_cpt > 0):
// bit k for key 64 * (it - run * chunks_per_run) + k of its run. Everything
// here is uniform over the wave, so it takes no vector work.
STA_HD unsigned long long chunk_pad_mask(const AttnParams& p, const KvRuns& kv, int chunks_per_run,
                                         int it) {
  const int run = it / chunks_per_run;
  const int rt = run / kv.oh, rh = run - rt * kv.oh;
  const int j = it - run * chunks_per_run;
  const int tw = j / p.pad_cpt, c = j - tw * p.pad_cpt;
  unsigned long long m = ~0ull;
  if ((kv.st + rt + 1) * p.ct > p.T) m &= p.pad_mask[0][c];
  if ((kv.sh + rh + 1) * p.ch > p.H) m &= p.pad_mask[1][c];
  if ((kv.sw + tw + 1) * p.cw > p.W) m &= p.pad_mask[2][c];
  return m;
}

// Raster token index of row `local` (tile-major order inside the tile) of
// query tile (qt, qh, qw).
STA_HD int tile_row_raster(const AttnParams& p, int qt, int qh, int qw, int local) {
  const int plane = p.ch * p.cw;
  const int lt = local / plane;
  const int rem = local - lt * plane;
  const int lh = rem / p.cw;
  const int lw = rem - lh * p.cw;
  return ((qt * p.ct + lt) * p.H + qh * p.ch + lh) * p.W + qw * p.cw + lw;
}

// Raster offset, relative to the run's first key, of key e of a window run
// (tile-major order within the run: tile along w, then the tile's tokens).
STA_HD int run_offset_raster(const AttnParams& p, int e) {
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
STA_HD Task decode_task(const AttnParams& p, int task, int D) {
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
  t.valid_rows = imin(ROWS, p.unit_rows - rb * ROWS);
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

// Walks the key chunks of a work item: chunk `it` covers keys
// row0(it) .. + BN of the head, of which nvalid(it) are inside the run.
struct ChunkWalk {
  int chunks_per_run, n_chunks, run_len, bn;
  KvRuns kv;
  bool dense;
  STA_HD void at(int it, int* row0, int* nvalid) const {
    const int run = it / chunks_per_run;
    const int c0 = (it - run * chunks_per_run) * bn;
    *row0 = (dense ? 0 : kv.run_start(run)) + c0;
    *nvalid = imin(bn, run_len - c0);
  }
  // Raster order, plane chunks: the raster token of the chunk's first key
  // (the chunk is one 64-row piece of one t-plane of one tile).
  STA_HD int at_plane(const AttnParams& p, int it) const {
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
  STA_HD void at_tile(int it, int tau, int* tile_row0, int* key_base,
                                          int* nvalid) const {
    const int run = it / chunks_per_run;
    const int c0 = (it - run * chunks_per_run) * bn;
    *key_base = c0 % tau;
    *tile_row0 = (dense ? 0 : kv.run_start(run)) + c0 - *key_base;
    *nvalid = imin(bn, run_len - c0);
  }
  // Raster order: the run's first raster token, the chunk's first key within
  // the run, and the number of valid keys.
  STA_HD void at_raster(const AttnParams& p, int it, int* base, int* c0,
                                            int* nvalid) const {
    const int run = it / chunks_per_run;
    *c0 = (it - run * chunks_per_run) * bn;
    *base = kv.run_start_raster(run, p.H, p.W, p.ct, p.ch, p.cw);
    *nvalid = imin(bn, run_len - *c0);
  }
};

template <int BN, bool DENSE>
STA_HD ChunkWalk make_walk(const Task& t, int S) {
  ChunkWalk cw;
  cw.kv = t.kv;
  cw.dense = DENSE;
  cw.run_len = DENSE ? S : t.kv.run_len;
  cw.bn = BN;
  cw.chunks_per_run = (cw.run_len + BN - 1) / BN;
  cw.n_chunks = (DENSE ? 1 : t.kv.runs) * cw.chunks_per_run;
  return cw;
}

// Host side: kernel parameters of an attention problem whose work items hold
// rows_per_item rows.
inline void fill_params(const AttnProblem& pr, int rows_per_item, AttnParams* p) {
  p->q = pr.q; p->k = pr.k; p->v = pr.v; p->out = pr.out;
  p->lse = pr.lse;
  p->n_cand = pr.dense ? 0 : pr.n_cand;
  p->lse_cand = pr.lse_cand;
  p->cand_stride = pr.cand_stride;
  for (int c = 0; c < kMaxRecallCand; ++c)
    for (int a = 0; a < 3; ++a) p->cand_omega[c][a] = c < p->n_cand ? pr.cand_omega[c][a] : 0;
  // rows per (batch, head) of the tensors: tile-major tensors of a padded
  // tile grid hold n_tiles * tau rows
  p->S = pr.dense || pr.raster ? pr.g.S : pr.g.S_pad;
  p->heads = pr.heads;
  p->dense = pr.dense ? 1 : 0;
  p->scale_log2 = pr.scale * kLog2e;
  if (pr.dense) {
    p->n_units = 1;
    p->unit_rows = pr.g.S;
    p->nt = p->nh = p->nw = 1;
    p->tau = pr.g.S;
    p->T = p->H = p->W = p->ct = p->ch = p->cw = 1;
    p->pad = 0;
    p->plane_cpt = p->plane_cpp = 0;
    p->pad_cpt = 0;
  } else {
    p->n_units = pr.g.n_tiles;
    p->unit_rows = pr.g.tau;
    p->nt = pr.g.nt; p->nh = pr.g.nh; p->nw = pr.g.nw;
    p->tau = pr.g.tau;
    p->T = pr.g.T; p->H = pr.g.H; p->W = pr.g.W;
    p->ct = pr.g.ct; p->ch = pr.g.ch; p->cw = pr.g.cw;
    p->pad = pr.g.padded;
    set_plane_chunks(p);
    set_pad_masks(p);
    for (int h = 0; h < pr.heads; ++h)
      for (int a = 0; a < 3; ++a) p->omega[h][a] = pr.omega[h][a];
  }
  p->row_blocks = (p->unit_rows + rows_per_item - 1) / rows_per_item;
  // one entry per 64-key chunk of the whole-volume walk
  p->cand_chunks = p->n_cand ? (int)((long long)p->n_units * ((p->tau + 63) / 64)) : 0;
  const long long tasks = (long long)pr.B * pr.heads * p->n_units * p->row_blocks;
  plan_tasks(p, tasks, pr.heads, pr.dense);
}

// Backward parameters beyond AttnParams.
struct BwdParams {
  const void* dout;    // dO, same shape and order as q
  const float* lse;    // [B][heads][S] forward log-sum-exp (natural log)
  float* delta;        // [B][heads][S] D = dO . O (written by delta_kernel)
  void* dq;
  void* dk;
  void* dv;
  float scale;
};

// Host side: parameters of a backward pass whose work items hold
// rows_per_item own rows (key rows or query rows).
inline void fill_bwd_params(const BwdProblem& pr, int rows_per_item, AttnParams* p, BwdParams* b) {
  const AttnProblem& a = pr.attn;
  p->q = a.q; p->k = a.k; p->v = a.v; p->out = a.out;
  p->lse = nullptr;
  p->n_cand = 0;
  p->cand_chunks = 0;
  p->lse_cand = nullptr;
  p->cand_stride = 0;
  p->S = a.raster ? a.g.S : a.g.S_pad;
  p->heads = a.heads;
  p->dense = 0;
  p->scale_log2 = a.scale * kLog2e;
  p->n_units = a.g.n_tiles;
  p->unit_rows = a.g.tau;
  p->nt = a.g.nt; p->nh = a.g.nh; p->nw = a.g.nw;
  p->tau = a.g.tau;
  p->T = a.g.T; p->H = a.g.H; p->W = a.g.W;
  p->pad = a.g.padded;
  p->ct = a.g.ct; p->ch = a.g.ch; p->cw = a.g.cw;
  set_plane_chunks(p);
  set_pad_masks(p);
  for (int h = 0; h < a.heads; ++h)
    for (int x = 0; x < 3; ++x) p->omega[h][x] = a.omega[h][x];
  p->row_blocks = (p->unit_rows + rows_per_item - 1) / rows_per_item;
  const long long tasks = (long long)a.B * a.heads * p->n_units * p->row_blocks;
  plan_tasks(p, tasks, a.heads, false);
  b->dout = pr.dout;
  b->lse = pr.lse;
  b->delta = pr.delta;
  b->dq = pr.dq; b->dk = pr.dk; b->dv = pr.dv;
  b->scale = a.scale;
}

// Work-item shapes (rows per item) the launchers use; the host-side bounds
// model takes them from here too.
#ifndef STA_CFG_WAVES
#define STA_CFG_WAVES 8
#endif
#ifndef STA_CFG_RB
#define STA_CFG_RB 3
#endif
#ifndef STA_CFG_BN
#define STA_CFG_BN 64
#endif
constexpr int kFwdBigRows = STA_CFG_WAVES * 16 * STA_CFG_RB;
// Rows of the items a split last round runs as (two groups of 4 waves of 16
// rows, each group taking half of the key chunks).
constexpr int kFwdTailRows = 64;
// Rows of the items of a one-pass window recall (4 waves of 32 rows).
constexpr int kRecallRows = 128;
// bf16 forward: the big shape when a unit is whole blocks of it, else 4 waves
// of 16 rows (units of at most 64 rows) or of 32 rows.
inline int fwd_bf16_rows(int unit_rows) {
  return unit_rows % kFwdBigRows == 0 ? kFwdBigRows : unit_rows <= 64 ? 64 : 128;
}
// float32 forward: 32 query rows an item, two lanes a row (half the head
// dimension each); every wave of the workgroup holds the same rows and takes
// every f32_key_splits(D)-th 32-key chunk of the window, and the waves'
// partial results are merged at the end.
constexpr int kF32Rows = 32;
constexpr int kF32BN = 32;         // keys per chunk
STA_HD constexpr int f32_key_splits(int D) { return D <= 64 ? 8 : 4; }
// bf16 backward, key side: 4 pairs of waves sharing 48 key rows when such
// items tile tau, else pairs sharing 32 key rows (tiles of at least 128
// tokens), else 4 waves of 16; query side: 4 waves of 32 query rows, else of
// 16.
inline int bwd_key_rows(int tau) {
  if (tau % 192 == 0) return 192;
  return tau >= 128 ? 128 : 64;
}
inline int bwd_query_rows(int tau) { return tau >= 128 ? 128 : 64; }

// Logical task of workgroup `bid`: consecutive logical tasks (the row blocks
// of one query tile, then neighbouring tiles that share most of their keys)
// run on the same XCD and share its L2.
STA_HD int task_of_block(const AttnParams& p, int bid) {
  const int x = bid % kXcds, r = bid / kXcds;
  if (p.tail_split) {
    // Tail launch: row block r % tail_split of the work item the XCD's round
    // tail_r0 + r / tail_split would have run, on the same XCD.
    const int mr = p.tail_r0 + r / p.tail_split;
    const int item = (mr / p.group) * (kXcds * p.group) + x * p.group + mr % p.group;
    return item * p.tail_split + r % p.tail_split;
  }
  return (r / p.group) * (kXcds * p.group) + x * p.group + r % p.group;
}

// Host side: the last round of work items. Under an equal-cost plan each XCD
// runs `group` items on cu_per_xcd CUs, one workgroup per CU; when group is
// not a multiple of cu_per_xcd the last round leaves most of the XCD idle for
// a whole item. If its items, cut into split = main_rows / tail_rows row
// blocks, fit two to a CU, the main launch stops before that round and `t`
// describes a second launch of tail_rows-row items that runs them side by
// side. Row block b of item i is item i * split + b of the tail launch (the
// same rows as under a plain tail_rows-row plan). Returns whether to split;
// *main_per_xcd is the main launch's workgroups per XCD either way.
inline bool plan_tail_split(const AttnProblem& pr, const AttnParams& m, int main_rows, int tail_rows,
                            int cu_per_xcd, AttnParams* t, int* main_per_xcd) {
  *main_per_xcd = m.per_xcd;
  if (cu_per_xcd <= 0 || m.group != m.per_xcd || m.group < cu_per_xcd) return false;
  if (tail_rows <= 0 || main_rows % tail_rows || m.unit_rows % main_rows) return false;
  const int rem = m.group % cu_per_xcd;
  const int split = main_rows / tail_rows;
  if (rem == 0 || (long long)rem * split > 2LL * cu_per_xcd) return false;
  fill_params(pr, tail_rows, t);
  if ((long long)t->n_tasks != (long long)m.n_tasks * split) return false;
  t->group = m.group;
  t->per_xcd = rem * split;
  t->tail_split = split;
  t->tail_r0 = m.group - rem;
  *main_per_xcd = m.group - rem;
  return true;
}

}  // namespace
}  // namespace sta
