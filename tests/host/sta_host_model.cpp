// Host-side bounds model of libsta -- test infrastructure.
//
// Built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
// together with the C-ABI layer (sta_api.cpp), whose device launchers are
// replaced here by a model: instead of launching, each launcher walks the
// exact grid the real one would launch (same kernel parameters, from
// fill_params / fill_bwd_params; same work-item shapes; same task decoding,
// window walk and row maps, from sta_plan.h) and checks that every row a
// workgroup would read or write lies inside its tensor, that every LDS index
// of the chunk staging stays inside its buffer, and that the 32-bit byte
// offsets of the direct-to-LDS loads stay below 2^31. The checks abort the
// program on the first violation (with the problem and the access named).
//
// main() then drives the C ABI: the five named workloads and small ones in
// both token orders (padded tile grids, ragged runs, per-head windows, the
// dense comparator, the backward, window recall) and a set of invalid calls
// that must be refused before any launch. Finally it runs the float32
// forward's index model on a padded grid directly (the API refuses that
// case) and reports where its unpadded row mapping would leave the tensor.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "sta.h"
#include "sta_kernels.h"
#include "sta_plan.h"

namespace {

using sta::AttnParams;
using sta::ChunkWalk;
using sta::Task;

struct Ctx {
  std::string what;     // the problem under test
  long long checks = 0;
  long long launches = 0;
  long long tail_launches = 0;   // forward launches whose last round ran as 64-row items
  long long recall_passes = 0;   // one-pass window recall launches
  long long pad_masks = 0;       // padded chunks whose precomputed token mask was checked
} g_ctx;

#define CHECK_ROW(row_, rows_, msg_)                                                         \
  do {                                                                                       \
    ++g_ctx.checks;                                                                          \
    if ((long long)(row_) < 0 || (long long)(row_) >= (long long)(rows_)) {                 \
      fprintf(stderr, "BOUNDS VIOLATION in %s: %s row %lld outside [0, %lld)\n",           \
              g_ctx.what.c_str(), msg_, (long long)(row_), (long long)(rows_));             \
      abort();                                                                               \
    }                                                                                        \
  } while (0)

#define CHECK(cond_, msg_)                                                                   \
  do {                                                                                       \
    ++g_ctx.checks;                                                                          \
    if (!(cond_)) {                                                                          \
      fprintf(stderr, "CHECK FAILED in %s: %s (%s)\n", g_ctx.what.c_str(), msg_, #cond_);   \
      abort();                                                                               \
    }                                                                                        \
  } while (0)

// Whether key `e` of run `run` of walk `w` is a token (the kernels' mask,
// chunk_real_keys, one key at a time).
bool key_real(const AttnParams& p, const ChunkWalk& w, int run, int e, bool pad) {
  if (!pad) return true;
  if (!sta::run_padded(p, w.kv, run)) return true;
  return e < w.run_len && sta::run_key_real(p, w.kv, run, e);
}

// Rows one chunk load (64 keys, as load_rows / load_rows_plane address
// them) reads; `rows` is the slice's row count. row_bytes: bytes per row of
// the streamed tensor (the byte offset of a lane's load must stay < 2^31).
void model_chunk(const AttnParams& p, const ChunkWalk& w, int it, bool raster, bool plane, bool pad,
                 long long rows, int row_bytes, int table_len, const char* what) {
  const int run = it / w.chunks_per_run;
  CHECK(run >= 0 && run < (w.dense ? 1 : w.kv.runs), "chunk index inside the walk");
  if (pad && p.pad_cpt > 0 && w.bn == 64) {
    // the kernels take the token mask of such a chunk from the plan's tables
    // (chunk_pad_mask): it must equal the per-key definition
    const unsigned long long m = sta::chunk_pad_mask(p, w.kv, w.chunks_per_run, it);
    const int j = it - run * w.chunks_per_run;
    for (int k = 0; k < 64; ++k)
      CHECK(((m >> k) & 1ull) == (key_real(p, w, run, j * 64 + k, pad) ? 1ull : 0ull),
            "precomputed chunk token mask");
    ++g_ctx.pad_masks;
  }
  if (plane) {
    const int row0 = w.at_plane(p, it);
    for (int key = 0; key < 64; ++key) {
      const int off = (key / p.cw) * p.W + key % p.cw;   // plane_lane_rows
      CHECK((long long)off * row_bytes + row_bytes <= (1LL << 31), "plane load offset below 2^31");
      CHECK_ROW((long long)row0 + off, rows, what);
    }
    return;
  }
  if (raster) {
    int base, c0, nv;
    w.at_raster(p, it, &base, &c0, &nv);
    CHECK(nv >= 1 && nv <= 64, "valid keys of a chunk");
    for (int key = 0; key < 64; ++key) {
      const int k = key < nv ? key : nv - 1;
      CHECK(c0 + k < table_len, "raster offset table index");
      int rel = sta::run_offset_raster(p, c0 + k);
      if (!key_real(p, w, run, c0 + k, pad)) rel = 0;
      CHECK((long long)rel * row_bytes + row_bytes <= (1LL << 31), "raster load offset below 2^31");
      CHECK_ROW((long long)base + rel, rows, what);
    }
    return;
  }
  int row0, kb = 0, nv;
  if (pad) {
    w.at_tile(it, p.tau, &row0, &kb, &nv);
  } else {
    w.at(it, &row0, &nv);
  }
  CHECK(nv >= 1 && nv <= 64, "valid keys of a chunk");
  for (int key = 0; key < 64; ++key) {
    const int k = key < nv ? key : nv - 1;
    int rel = kb + k;
    if (pad && !key_real(p, w, run, (it - run * w.chunks_per_run) * 64 + k, pad)) rel = 0;
    CHECK((long long)rel * row_bytes + row_bytes <= (1LL << 31), "tile-major load offset below 2^31");
    CHECK_ROW((long long)row0 + rel, rows, what);
  }
}

// Own rows of a work item (map_rows): rows r = 0 .. ROWS-1 of the item; a
// row that exists is read and written, one that does not reads the unit's
// first row and is never written.
template <int ROWS>
void model_own_rows(const AttnParams& p, const Task& t, bool raster, long long rows, const char* what) {
  for (int r = 0; r < ROWS; ++r) {
    const bool ok = r < t.valid_rows && (!p.pad || sta::tile_row_real(p, t.qt, t.qh, t.qw, t.local0 + r));
    const int local = ok ? t.local0 + r : 0;
    const long long tok = raster ? sta::tile_row_raster(p, t.qt, t.qh, t.qw, local) : t.row0 - t.local0 + local;
    CHECK_ROW(tok, rows, what);
  }
}

// Head bases: every (batch, head) slice starts inside the tensor.
void check_head(const AttnParams& p, const Task& t, int D, long long total_rows) {
  CHECK(t.head_base % D == 0, "head base is a whole row");
  CHECK_ROW(t.head_base / D, total_rows, "head base");
  CHECK_ROW(t.head_base / D + p.S - 1, total_rows, "head end");
}

// The bf16 forward (attn_bf16_kernel) and its dense form: every workgroup of
// the grid of one launch planned in p; each task it runs is marked in seen.
// groups = 2: the key-split configuration (the last round's 64-row items):
// two groups of waves on the same rows, group g taking chunks g, g + 2, ...
// at steps 0, 1, ..., each with its own double-buffered K and V, all of it
// (with the raster table) within the 160 KB of LDS a workgroup can hold.
template <int ROWS>
void model_bf16_launch(const sta::AttnProblem& pr, const AttnParams& p, long long grid,
                       std::vector<char>& seen, int groups = 1) {
  const int D = pr.head_dim;
  const long long total_rows = (long long)pr.B * pr.heads * p.S;
  const bool full = [&] {
    if (pr.dense) return pr.g.S % 64 == 0;
    if (pr.g.padded) return false;
    for (int h = 0; h < pr.heads; ++h)
      if ((pr.omega[h][2] * pr.g.tau) % 64) return false;
    return true;
  }();
  const bool plane = pr.raster && !pr.dense && full && p.plane_cpt > 0;
  int table_len = 0;
  for (int h = 0; h < pr.heads && !pr.dense; ++h)
    table_len = pr.omega[h][2] * pr.g.tau > table_len ? pr.omega[h][2] * pr.g.tau : table_len;
  CHECK(!pr.raster || pr.dense || plane || table_len <= sta::kMaxRasterRun, "raster table fits LDS");
  const int k_row_bytes = pr.qk_fp8 ? D : 2 * D;
  CHECK(grid <= (1LL << 31) - 1, "grid fits the launch");
  for (long long bid = 0; bid < grid; ++bid) {
    const int task = sta::task_of_block(p, (int)bid);
    if (task >= p.n_tasks) continue;
    CHECK(task >= 0 && !seen[task], "each task exactly once");
    seen[task] = 1;
    const Task t = sta::decode_task<ROWS>(p, task, D);
    check_head(p, t, D, total_rows);
    model_own_rows<ROWS>(p, t, pr.raster && !pr.dense, p.S, "query");
    const ChunkWalk w = pr.dense ? sta::make_walk<64, true>(t, p.S) : sta::make_walk<64, false>(t, p.S);
    if (p.n_cand > 0) {
      // every chunk of the whole-volume walk has an entry in the candidate
      // table, and the candidate windows' rows are written like lse's
      CHECK(w.n_chunks <= p.cand_chunks, "candidate table covers the walk");
      CHECK(p.cand_stride >= total_rows, "each candidate's rows have a slot of their own");
    }
    const int steps = (w.n_chunks + groups - 1) / groups;
    int loaded = 0;
    for (int st = 0; st < steps; ++st)
      for (int grp = 0; grp < groups; ++grp) {
        const int it = st * groups + grp;
        if (it >= w.n_chunks) continue;   // the group only keeps the step's barriers
        model_chunk(p, w, it, pr.raster && !pr.dense, plane, p.pad, p.S, k_row_bytes, table_len, "key");
        ++loaded;
      }
    CHECK(loaded == w.n_chunks, "every chunk of the walk runs exactly once");
  }
  if (groups > 1) {
    const long long v_bytes = pr.lse_only ? 16 : 64LL * 2 * D;
    const long long stat = 2LL * groups * (64LL * k_row_bytes + v_bytes);
    const bool table = pr.raster && !pr.dense && !plane;
    CHECK(stat + (table ? 4LL * table_len : 0) <= 163840, "key-split LDS within 160 KB");
    CHECK(pr.lse_only || 4LL * (ROWS / 16) * (D / 4) * 64 <= groups * 64LL * 2 * D, "merge output fits the V buffers");
  }
  ++g_ctx.launches;
}

// Compute units per XCD the model plans for (MI355X: 256 over 8 XCDs).
constexpr int kModelCuPerXcd = 32;

// The bf16 forward as the launcher issues it: the main launch, and for whole-
// tile items a second launch of the last round cut into 64-row items when
// plan_tail_split asks for it. Every row block must run exactly once.
template <int ROWS>
void model_bf16_forward(const sta::AttnProblem& pr) {
  AttnParams p, tp;
  sta::fill_params(pr, ROWS, &p);
  int main_per_xcd = p.per_xcd;
  const bool tail = ROWS == sta::kFwdBigRows &&
                    sta::plan_tail_split(pr, p, ROWS, sta::kFwdTailRows, kModelCuPerXcd, &tp, &main_per_xcd);
  std::vector<char> seen(p.n_tasks, 0);
  model_bf16_launch<ROWS>(pr, p, (long long)main_per_xcd * sta::kXcds, seen);
  if (!tail) {
    CHECK(p.n_tasks <= (long long)p.per_xcd * sta::kXcds, "grid covers every task");
    for (int i = 0; i < p.n_tasks; ++i) CHECK(seen[i], "every task has a workgroup");
    return;
  }
  ++g_ctx.tail_launches;
  std::vector<char> tseen(tp.n_tasks, 0);
  model_bf16_launch<sta::kFwdTailRows>(pr, tp, (long long)tp.per_xcd * sta::kXcds, tseen, 2);
  for (int i = 0; i < p.n_tasks; ++i) {
    int parts = 0;
    for (int b = 0; b < tp.tail_split; ++b) parts += tseen[(size_t)i * tp.tail_split + b];
    CHECK(seen[i] ? parts == 0 : parts == tp.tail_split,
          "each item once: whole in the main launch or all its row blocks in the tail launch");
  }
}

// The float32 forward (attn_f32_kernel): 32 query rows an item, lane l of
// every wave on row l % 32 (half the dimensions each); wave w stages chunks
// w, w + KS, ... of 32 keys in its own K and V buffers of one LDS array, which
// the merge then reuses as [KS][D][32] floats.
template <int D>
void model_f32_forward(const sta::AttnProblem& pr) {
  constexpr int KS = sta::f32_key_splits(D);
  constexpr int D4 = D / 4;
  constexpr int kStage = KS * 2 * sta::kF32BN * D4;
  constexpr int kMerge = KS * D * sta::kF32Rows / 4;
  constexpr int kLds = kStage > kMerge ? kStage : kMerge;   // float4
  AttnParams p;
  sta::fill_params(pr, sta::kF32Rows, &p);
  const long long total_rows = (long long)pr.B * pr.heads * p.S;
  const bool raster = pr.raster && !pr.dense;
  const long long grid = (long long)p.per_xcd * sta::kXcds;
  for (long long bid = 0; bid < grid; ++bid) {
    const int task = sta::task_of_block(p, (int)bid);
    if (task >= p.n_tasks) continue;
    const Task t = sta::decode_task<sta::kF32Rows>(p, task, D);
    check_head(p, t, D, total_rows);
    for (int lane = 0; lane < 64; ++lane) {
      const int row = lane % sta::kF32Rows, half = lane / sta::kF32Rows;
      const bool row_ok = row < t.valid_rows;
      const int my_row = row_ok ? row : 0;
      const long long q_tok = raster ? sta::tile_row_raster(p, t.qt, t.qh, t.qw, t.local0 + my_row)
                                     : (long long)t.row0 + my_row;
      CHECK_ROW(q_tok, p.S, row_ok ? "f32 query (read and written)" : "f32 query (read)");
      for (int w = 0; w < KS; ++w)
        for (int d = 0; d < D / 2; ++d)
          CHECK((w * D + half * (D / 2) + d) * sta::kF32Rows + row < 4 * kLds, "f32 merge index");
      for (int wave = 0; wave < KS; ++wave)
        for (int dd = 0; dd < D / KS / 2; ++dd) {
          const int d = (2 * wave + half) * (D / KS / 2) + dd;
          CHECK(d < D, "f32 stored dimension");
          for (int w = 0; w < KS; ++w) CHECK((w * D + d) * sta::kF32Rows + row < 4 * kLds, "f32 merge read");
        }
      for (int j = 0; j < sta::kF32BN; ++j)
        for (int d4 = 0; d4 < D4 / 2; ++d4) CHECK(half * (D4 / 2) + j * D4 + d4 < sta::kF32BN * D4, "f32 operand read");
    }
    const int cpr = (t.kv.run_len + sta::kF32BN - 1) / sta::kF32BN;
    const int n_chunks = t.kv.runs * cpr;
    for (int wave = 0; wave < KS; ++wave)
      for (int c = wave; c < n_chunks; c += KS) {
        const int run = c / cpr;
        const int c0 = (c - run * cpr) * sta::kF32BN;
        CHECK(c0 < t.kv.run_len, "f32 chunk inside its run");
        const int nvalid = sta::imin(sta::kF32BN, t.kv.run_len - c0);
        const long long kv0 = raster ? t.kv.run_start_raster(run, p.H, p.W, p.ct, p.ch, p.cw)
                                     : t.kv.run_start(run);
        for (int i = 0; i < sta::kF32BN * D4; ++i) {
          const int key = i / D4;
          CHECK(wave * (2 * sta::kF32BN * D4) + sta::kF32BN * D4 + i < kLds, "f32 LDS staging index");
          if (key < nvalid) {
            const long long tok = kv0 + (raster ? sta::run_offset_raster(p, c0 + key) : c0 + key);
            CHECK_ROW(tok, p.S, "f32 key");
          }
        }
      }
  }
  ++g_ctx.launches;
}

// The float32 backward (bwd_f32_dkdv_kernel, bwd_f32_dq_kernel): 32 own
// rows an item, lane l of every wave on row l % 32; wave w stages chunks w,
// w + KS, ... of 32 streamed rows (and, on the key side, their lse and D);
// the merge reuses the staging array as [KS][D][32] (query side) or
// [KS][2][D][32] (key side) floats.
template <int D>
void model_f32_backward(const sta::BwdProblem& pb) {
  const sta::AttnProblem& a = pb.attn;
  constexpr int KS = sta::f32_key_splits(D);
  constexpr int D4 = D / 4;
  constexpr int R = sta::kF32Rows;
  constexpr int kStage = KS * 2 * sta::kF32BN * D4;
  const long long total_rows = (long long)a.B * a.heads * (a.raster ? a.g.S : a.g.S_pad);
  for (int side = 0; side < 2; ++side) {
    const bool keys = side == 0;
    const int kMerge = KS * (keys ? 2 : 1) * D * R / 4;
    const int kLds = kStage > kMerge ? kStage : kMerge;
    AttnParams p;
    sta::BwdParams b;
    sta::fill_bwd_params(pb, R, &p, &b);
    const long long grid = (long long)p.per_xcd * sta::kXcds;
    for (long long bid = 0; bid < grid; ++bid) {
      const int task = sta::task_of_block(p, (int)bid);
      if (task >= p.n_tasks) continue;
      const Task t = keys ? sta::decode_task<R, true>(p, task, D) : sta::decode_task<R>(p, task, D);
      check_head(p, t, D, total_rows);
      for (int lane = 0; lane < 64; ++lane) {
        const int row = lane % R, half = lane / R;
        const int r = row < t.valid_rows ? row : 0;
        const long long tok = a.raster ? sta::tile_row_raster(p, t.qt, t.qh, t.qw, t.local0 + r)
                                       : (long long)t.row0 + r;
        CHECK_ROW(tok, p.S, keys ? "f32 own key" : "f32 own query");
        for (int w = 0; w < KS; ++w)
          for (int m = 0; m < (keys ? 2 : 1); ++m)
            for (int d = 0; d < D / 2; ++d)
              CHECK(((w * (keys ? 2 : 1) + m) * D + half * (D / 2) + d) * R + row < 4 * kLds, "f32 backward merge index");
        for (int dd = 0; dd < D / KS / 2; ++dd) CHECK((2 * (KS - 1) + half) * (D / KS / 2) + dd < D, "f32 stored dimension");
      }
      const int cpr = (t.kv.run_len + sta::kF32BN - 1) / sta::kF32BN;
      const int n_chunks = t.kv.runs * cpr;
      for (int wave = 0; wave < KS; ++wave)
        for (int c = wave; c < n_chunks; c += KS) {
          const int run = c / cpr;
          const int c0 = (c - run * cpr) * sta::kF32BN;
          CHECK(c0 < t.kv.run_len, "f32 chunk inside its run");
          const int nvalid = sta::imin(sta::kF32BN, t.kv.run_len - c0);
          const long long row0 = a.raster ? t.kv.run_start_raster(run, p.H, p.W, p.ct, p.ch, p.cw)
                                          : t.kv.run_start(run);
          for (int i = 0; i < sta::kF32BN * D4; ++i) {
            CHECK(wave * (2 * sta::kF32BN * D4) + sta::kF32BN * D4 + i < kLds, "f32 backward staging index");
            const int key = i / D4;
            if (key < nvalid)
              CHECK_ROW(row0 + (a.raster ? sta::run_offset_raster(p, c0 + key) : c0 + key), p.S,
                        keys ? "f32 streamed query (q, dO, lse, D)" : "f32 streamed key (k, v)");
          }
        }
    }
    ++g_ctx.launches;
  }
}

// The backward's two passes: key side (own key rows, walking the query tiles
// whose window holds the key tile) and query side (own query rows, walking the
// window), with their work-item shapes.
template <int KROWS, int QROWS>
void model_bf16_backward(const sta::BwdProblem& pb) {
  const sta::AttnProblem& a = pb.attn;
  const int D = a.head_dim;
  for (int side = 0; side < 2; ++side) {
    AttnParams p;
    sta::BwdParams b;
    sta::fill_bwd_params(pb, side == 0 ? KROWS : QROWS, &p, &b);
    const long long total_rows = (long long)a.B * a.heads * p.S;
    int table_len = 0;
    for (int h = 0; h < a.heads; ++h) {
      int len = a.omega[h][2];
      if (side == 0) {
        len = 0;
        for (int j = 0; j < a.g.nw; ++j) {
          int lo, hi;
          sta::window_inverse(j, a.g.nw, a.omega[h][2], &lo, &hi);
          len = hi - lo + 1 > len ? hi - lo + 1 : len;
        }
      }
      table_len = len * a.g.tau > table_len ? len * a.g.tau : table_len;
    }
    const long long grid = (long long)p.per_xcd * sta::kXcds;
    for (long long bid = 0; bid < grid; ++bid) {
      const int task = sta::task_of_block(p, (int)bid);
      if (task >= p.n_tasks) continue;
      const Task t = side == 0 ? sta::decode_task<KROWS, true>(p, task, D) : sta::decode_task<QROWS>(p, task, D);
      check_head(p, t, D, total_rows);
      if (side == 0)
        model_own_rows<KROWS>(p, t, a.raster, p.S, "own key");
      else
        model_own_rows<QROWS>(p, t, a.raster, p.S, "own query");
      const ChunkWalk w = sta::make_walk<64, false>(t, p.S);
      for (int it = 0; it < w.n_chunks; ++it)
        model_chunk(p, w, it, a.raster, false, p.pad, p.S, 2 * D, table_len,
                    side == 0 ? "streamed query" : "streamed key");
    }
    ++g_ctx.launches;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// The launchers sta_api.cpp calls, replaced by the model
// ---------------------------------------------------------------------------

namespace sta {

int launch_reorder(const void*, void*, int BH, int row_bytes, const Geometry& g, bool, void*) {
  CHECK(BH > 0 && row_bytes % 16 == 0 && g.S <= g.S_pad, "reorder arguments");
  ++g_ctx.launches;
  return 0;
}

int launch_kv_tiles(int*, int*, int heads, const Geometry& g, const uint16_t (*omega)[3], int max_kv,
                    bool transposed, void*) {
  CHECK(heads >= 1 && heads <= STA_MAX_HEADS && max_kv >= 1, "tile-list arguments");
  for (int h = 0; h < heads; ++h)
    CHECK(omega[h][0] >= 1 && omega[h][0] <= g.nt && omega[h][1] <= g.nh && omega[h][2] <= g.nw,
          "window inside the tile grid");
  (void)transposed;
  ++g_ctx.launches;
  return 0;
}

int launch_attention(const AttnProblem& pr, void*) {
  if (pr.qk_fp8 && !(pr.dtype == STA_BF16 && pr.head_dim == 128)) return STA_ERR_UNSUPPORTED;
  if (pr.head_dim != 64 && pr.head_dim != 128) return STA_ERR_UNSUPPORTED;
  if (pr.n_cand > 0) {
    // one-pass window recall: the launcher's rules (bf16 log-sum-exp only,
    // whole 64-key chunks, tile-major or plane chunks, a table that fits)
    if (pr.dtype != STA_BF16 || pr.dense || !pr.lse_only) return STA_ERR_UNSUPPORTED;
    AttnParams p;
    sta::fill_params(pr, 64, &p);
    bool full = !pr.g.padded;
    for (int h = 0; h < pr.heads; ++h) full = full && (pr.omega[h][2] * pr.g.tau) % 64 == 0;
    if (!full || (pr.raster && p.plane_cpt == 0) || p.cand_chunks > sta::kMaxRecallTable)
      return STA_ERR_UNSUPPORTED;
    CHECK(pr.n_cand <= sta::kMaxRecallCand, "candidates fit the kernel");
    ++g_ctx.recall_passes;
    model_bf16_forward<sta::kRecallRows>(pr);
    return 0;
  }
  if (pr.dtype == STA_F32) {
    CHECK(!(pr.g.padded && !pr.dense), "float32 attention never reaches a padded grid");
    if (pr.head_dim == 64) model_f32_forward<64>(pr); else model_f32_forward<128>(pr);
    return 0;
  }
  const int rows = fwd_bf16_rows(pr.dense ? pr.g.S : pr.g.tau);
  if (rows == kFwdBigRows) model_bf16_forward<kFwdBigRows>(pr);
  else if (rows == 64) model_bf16_forward<64>(pr);
  else model_bf16_forward<128>(pr);
  return 0;
}

int launch_backward(const BwdProblem& pb, void*) {
  const AttnProblem& a = pb.attn;
  if (a.head_dim != 64 && a.head_dim != 128) return STA_ERR_UNSUPPORTED;
  CHECK(pb.delta != nullptr, "the D workspace is set");
  if (a.dtype == STA_F32) {
    CHECK(!a.g.padded, "float32 backward never reaches a padded grid");
    if (a.head_dim == 64) model_f32_backward<64>(pb); else model_f32_backward<128>(pb);
    return 0;
  }
  const int kr = bwd_key_rows(a.g.tau), qr = bwd_query_rows(a.g.tau);
  if (kr == 192 && qr == 128) model_bf16_backward<192, 128>(pb);
  else if (kr == 128 && qr == 128) model_bf16_backward<128, 128>(pb);
  else if (kr == 64 && qr == 64) model_bf16_backward<64, 64>(pb);
  else CHECK(false, "known backward shapes");
  return 0;
}

int launch_recall_reduce(const float*, const float*, float*, int BH, int S, int n_cand, int c, void*) {
  CHECK(BH > 0 && S > 0 && c >= 0 && c < n_cand, "recall reduction arguments");
  ++g_ctx.launches;
  return 0;
}

// A fixed stand-in address for the static scratch (never dereferenced here).
int noalloc_scratch(float** ptr) {
  *ptr = reinterpret_cast<float*>(uintptr_t(1) << 44);
  return 0;
}

const char* hip_error_string(int) { return "modelled launch"; }

}  // namespace sta

// ---------------------------------------------------------------------------
// Driver
// ---------------------------------------------------------------------------

namespace {

// Never-dereferenced device addresses, far apart so that no two buffers
// overlap (each slot 2^36 bytes).
const void* slot(int i) { return reinterpret_cast<const void*>((uintptr_t)(i + 1) << 36); }
void* wslot(int i) { return reinterpret_cast<void*>((uintptr_t)(i + 1) << 36); }

struct Problem {
  const char* name;
  int B, heads, d, T, H, W;
  int tile[3];
  std::vector<int> windows;   // heads * 3 tokens
  int dtype;
};

int expect(int rc, int want, const char* call) {
  if (rc != want) {
    fprintf(stderr, "UNEXPECTED STATUS in %s: %s returned %d, expected %d (%s)\n", g_ctx.what.c_str(),
            call, rc, want, sta_last_error());
    abort();
  }
  return rc;
}

void run_valid(const Problem& pr) {
  const int* t = pr.tile;
  const int* w = pr.windows.data();
  const float scale = 0.125f;
  for (int order = 0; order < 2; ++order) {
    g_ctx.what = std::string(pr.name) + (order ? " raster" : " tile-major");
    const bool f32_padded = pr.dtype == STA_F32 && (pr.T % t[0] || pr.H % t[1] || pr.W % t[2]);
    const int want = f32_padded ? STA_ERR_UNSUPPORTED : STA_OK;
    if (order == 0) {
      expect(sta_reorder_tiles(slot(0), wslot(1), pr.B, pr.heads, pr.d, pr.T, pr.H, pr.W, t, pr.dtype, nullptr), 0, "sta_reorder_tiles");
      expect(sta_forward(slot(0), slot(1), slot(2), wslot(3), pr.B, pr.heads, pr.d, pr.T, pr.H, pr.W, t, w, scale, pr.dtype, nullptr), want, "sta_forward");
    } else {
      const int rc = sta_forward_raster(slot(0), slot(1), slot(2), wslot(3), pr.B, pr.heads, pr.d, pr.T, pr.H, pr.W, t, w, scale, pr.dtype, nullptr);
      if (rc != STA_ERR_UNSUPPORTED || !strstr(sta_last_error(), "raster")) expect(rc, want, "sta_forward_raster");
    }
    int rc = sta_forward_lse(slot(0), slot(1), slot(2), wslot(3), reinterpret_cast<float*>(wslot(4)), pr.B, pr.heads, pr.d, pr.T, pr.H, pr.W, t, w, scale, pr.dtype, order, nullptr);
    if (rc != STA_ERR_UNSUPPORTED || !strstr(sta_last_error(), "raster")) expect(rc, want, "sta_forward_lse");
    rc = sta_backward(slot(0), slot(1), slot(2), slot(3), slot(4), reinterpret_cast<const float*>(slot(5)), wslot(6), wslot(7), wslot(8), reinterpret_cast<float*>(wslot(9)), pr.B, pr.heads, pr.d, pr.T, pr.H, pr.W, t, w, scale, pr.dtype, order, nullptr);
    if (rc != STA_ERR_UNSUPPORTED || !strstr(sta_last_error(), "raster")) expect(rc, want, "sta_backward");
    if (pr.dtype == STA_BF16 && pr.d == 128) {
      rc = sta_forward_fp8(slot(0), slot(1), slot(2), wslot(3), pr.B, pr.heads, pr.d, pr.T, pr.H, pr.W, t, w, scale, 0.5f, 0.25f, order, nullptr);
      if (rc != STA_ERR_UNSUPPORTED || !strstr(sta_last_error(), "raster")) expect(rc, 0, "sta_forward_fp8");
      rc = sta_forward_fp8_lse(slot(0), slot(1), slot(2), wslot(3), reinterpret_cast<float*>(wslot(4)), pr.B, pr.heads, pr.d, pr.T, pr.H, pr.W, t, w, scale, 0.5f, 0.25f, order, nullptr);
      if (rc != STA_ERR_UNSUPPORTED || !strstr(sta_last_error(), "raster")) expect(rc, 0, "sta_forward_fp8_lse");
    }
    const int cands[6] = {w[0], w[1], w[2], t[0], t[1], t[2]};
    const bool padded = pr.T % t[0] || pr.H % t[1] || pr.W % t[2];
    const int want_recall = f32_padded || (padded && order == 0) ? STA_ERR_UNSUPPORTED : STA_OK;
    rc = sta_window_recall(slot(0), slot(1), reinterpret_cast<float*>(wslot(2)), reinterpret_cast<float*>(wslot(3)), pr.B, pr.heads, pr.d, pr.T, pr.H, pr.W, t, cands, 2, scale, pr.dtype, order, nullptr);
    if (rc != STA_ERR_UNSUPPORTED || !strstr(sta_last_error(), "raster")) expect(rc, want_recall, "sta_window_recall");
    if (pr.dtype == STA_BF16 && pr.d == 128) {
      rc = sta_window_recall_fp8(slot(0), slot(1), reinterpret_cast<float*>(wslot(2)), reinterpret_cast<float*>(wslot(3)), pr.B, pr.heads, pr.d, pr.T, pr.H, pr.W, t, cands, 2, scale, 0.5f, 0.25f, order, nullptr);
      if (rc != STA_ERR_UNSUPPORTED || !strstr(sta_last_error(), "raster")) expect(rc, want_recall, "sta_window_recall_fp8");
    }
  }
  // the dense comparator once at the large shape, on every small one
  if ((long long)pr.T * pr.H * pr.W > 20000 && strcmp(pr.name, "sta_30x48x80_whole_volume") != 0) return;
  g_ctx.what = std::string(pr.name) + " dense";
  expect(sta_full_attention(slot(0), slot(1), slot(2), wslot(3), pr.B, pr.heads, pr.d, pr.T * pr.H * pr.W, 0.1f, pr.dtype, nullptr), 0, "sta_full_attention");
}

std::vector<int> same(int heads, int a, int b, int c) {
  std::vector<int> v;
  for (int h = 0; h < heads; ++h) { v.push_back(a); v.push_back(b); v.push_back(c); }
  return v;
}

void run_invalid() {
  g_ctx.what = "invalid calls";
  const int t[3] = {6, 8, 8};
  const int w[3] = {18, 24, 24};
  const int bad_w[3] = {18, 24, 25};
  std::vector<int> many = same(STA_MAX_HEADS + 1, 18, 24, 24);
  expect(sta_forward(nullptr, slot(1), slot(2), wslot(3), 1, 1, 128, 30, 48, 80, t, w, 0.1f, 0, nullptr), STA_ERR_INVALID_ARG, "NULL q");
  expect(sta_forward(slot(0), slot(1), slot(2), wslot(3), 1, 1, 128, 30, 48, 80, t, bad_w, 0.1f, 0, nullptr), STA_ERR_INVALID_ARG, "window not whole tiles");
  expect(sta_forward(slot(0), slot(1), slot(2), wslot(3), 1, 1, 128, 30, 48, 80, nullptr, w, 0.1f, 0, nullptr), STA_ERR_INVALID_ARG, "NULL tile");
  expect(sta_forward(slot(0), slot(1), slot(2), wslot(3), 1, 1, 96, 30, 48, 80, t, w, 0.1f, 0, nullptr), STA_ERR_UNSUPPORTED, "head_dim 96");
  expect(sta_forward(slot(0), slot(1), slot(2), wslot(3), 1, 1, 128, 30, 48, 80, t, w, -1.0f, 0, nullptr), STA_ERR_INVALID_ARG, "negative scale");
  expect(sta_forward(slot(0), slot(1), slot(2), wslot(1), 1, 1, 128, 30, 48, 80, t, w, 0.1f, 0, nullptr), STA_ERR_INVALID_ARG, "out aliases k");
  expect(sta_forward(slot(0), slot(1), slot(2), wslot(3), 1, STA_MAX_HEADS + 1, 128, 30, 48, 80, t, many.data(), 0.1f, 0, nullptr), STA_ERR_INVALID_ARG, "too many heads");
  expect(sta_full_attention(slot(0), slot(1), slot(2), wslot(3), 1, STA_MAX_HEADS + 1, 128, 1024, 0.1f, 0, nullptr), STA_ERR_INVALID_ARG, "dense, too many heads");
  expect(sta_full_attention(slot(0), slot(1), slot(2), wslot(3), 1, 1, 128, 0, 0.1f, 0, nullptr), STA_ERR_INVALID_ARG, "dense, S = 0");
  expect(sta_kv_tiles(nullptr, reinterpret_cast<int*>(wslot(1)), 1, 30, 48, 80, t, w, 27, nullptr), STA_ERR_INVALID_ARG, "NULL list");
  expect(sta_kv_tiles(reinterpret_cast<int*>(wslot(0)), reinterpret_cast<int*>(wslot(1)), 1, 30, 48, 80, t, w, 26, nullptr), STA_ERR_INVALID_ARG, "short list");
  expect(sta_tile_list_len(1, 30, 48, 80, t, w, 1), 80, "transposed list length");
  expect(sta_tile_list_len(1, 30, 48, 80, t, bad_w, 0), STA_ERR_INVALID_ARG, "list length, bad window");
  expect((int)sta_kv_pair_count(1, 30, 48, 80, t, w), 8100, "pair count");
  expect(sta_reorder_tiles(slot(0), wslot(0), 1, 1, 128, 30, 48, 80, t, 0, nullptr), STA_ERR_INVALID_ARG, "in-place reorder");
  const int f32t[3] = {2, 4, 4}, f32w[3] = {4, 4, 4};
  expect(sta_forward(slot(0), slot(1), slot(2), wslot(3), 1, 1, 64, 5, 6, 7, f32t, f32w, 0.1f, STA_F32, nullptr), STA_ERR_UNSUPPORTED, "float32 on a padded grid");
  std::vector<int> heads73 = same(73, 18, 24, 24);
  expect(sta_backward_noalloc(slot(0), slot(1), slot(2), slot(3), slot(4), reinterpret_cast<const float*>(slot(5)), wslot(6), wslot(7), wslot(8), 1, 73, 128, 30, 48, 80, t, heads73.data(), 0.1f, 0, 1, nullptr), STA_ERR_INVALID_ARG, "no-alloc beyond its scratch");
  std::vector<int> heads72 = same(72, 18, 24, 24);
  expect(sta_backward_noalloc(slot(0), slot(1), slot(2), slot(3), slot(4), reinterpret_cast<const float*>(slot(5)), wslot(6), wslot(7), wslot(8), 1, 72, 128, 30, 48, 80, t, heads72.data(), 0.1f, 0, 1, nullptr), 0, "no-alloc within its scratch");
}

}  // namespace

int main() {
  std::vector<Problem> problems = {
      {"tiny_f32_12x16x16_w12", 1, 2, 64, 12, 16, 16, {4, 4, 4}, same(2, 12, 12, 12), STA_F32},
      // the 30x48x80 workloads with fewer heads (the index arithmetic of a
      // head does not depend on how many there are; the head bases do, and
      // B = 2 keeps the last slice's rows at the tensor's end)
      {"sta_30x48x80_w18x24x24", 2, 2, 128, 30, 48, 80, {6, 8, 8}, same(2, 18, 24, 24), STA_BF16},
      {"sta_30x48x80_w30x40x40", 1, 2, 128, 30, 48, 80, {6, 8, 8}, same(2, 30, 40, 40), STA_BF16},
      {"sta_30x48x80_whole_volume", 1, 1, 128, 30, 48, 80, {6, 8, 8}, same(1, 30, 48, 80), STA_BF16},
      {"mixed_windows", 1, 4, 128, 30, 48, 80, {6, 8, 8},
       {18, 24, 24, 18, 40, 40, 30, 24, 24, 30, 40, 40}, STA_BF16},
      {"padded_tile32_d64", 2, 3, 64, 5, 6, 7, {2, 4, 4}, {4, 4, 4, 2, 8, 8, 6, 8, 8}, STA_BF16},
      {"padded_tile96_d128", 2, 2, 128, 7, 12, 20, {3, 4, 8}, {6, 8, 16, 9, 12, 24}, STA_BF16},
      {"padded_tile384", 2, 2, 128, 10, 20, 30, {6, 8, 8}, {6, 16, 16, 12, 24, 24}, STA_BF16},
      {"padded_tile192_items", 2, 2, 128, 11, 9, 13, {4, 4, 12}, {8, 8, 12, 12, 12, 24}, STA_BF16},
      {"padded_tile384_items", 2, 1, 128, 13, 17, 19, {6, 8, 8}, {18, 24, 24}, STA_BF16},
      // the tile grid of the 30x48x80 workloads, padded (a one-plane last
      // t-tile), at 24 heads: the last round runs as key-split 64-row items
      {"padded_25x47x79_w6x24x24", 1, 24, 128, 25, 47, 79, {6, 8, 8}, same(24, 6, 24, 24), STA_BF16},
      {"ragged_tile48", 2, 2, 128, 9, 8, 12, {3, 4, 4}, {3, 4, 4, 6, 4, 8}, STA_BF16},
      {"image_2d_tile8x8", 1, 2, 128, 1, 32, 48, {1, 8, 8}, {1, 24, 24, 1, 32, 48}, STA_BF16},
      {"even_windows", 1, 2, 64, 8, 16, 16, {2, 4, 4}, {4, 8, 8, 8, 8, 4}, STA_BF16},
      {"f32_tile32_padded", 2, 2, 64, 5, 6, 7, {2, 4, 4}, {4, 4, 4, 6, 8, 8}, STA_F32},
      {"f32_d128", 1, 2, 128, 12, 16, 16, {4, 4, 4}, {4, 8, 8, 12, 16, 16}, STA_F32},
  };
  for (const Problem& pr : problems) run_valid(pr);
  run_invalid();

  // The float32 forward on the padded grid the API refuses (volume 5x6x7,
  // tile 2x4x4, d = 64, B = 2), modelled directly with its launch geometry:
  // how far its unpadded row mapping reaches past the volume.
  {
    sta::AttnProblem pr;
    memset(&pr, 0, sizeof(pr));
    pr.B = 2; pr.heads = 2; pr.head_dim = 64; pr.dtype = STA_F32; pr.scale = 0.125f;
    pr.g.T = 5; pr.g.H = 6; pr.g.W = 7; pr.g.ct = 2; pr.g.ch = 4; pr.g.cw = 4;
    pr.g.nt = 3; pr.g.nh = 2; pr.g.nw = 2; pr.g.n_tiles = 12; pr.g.tau = 32;
    pr.g.S = 210; pr.g.S_pad = 384; pr.g.padded = 1;
    const int om[2][3] = {{2, 1, 1}, {3, 2, 2}};
    for (int h = 0; h < 2; ++h)
      for (int a = 0; a < 3; ++a) pr.omega[h][a] = (uint16_t)om[h][a];
    for (int raster = 0; raster < 2; ++raster) {
      pr.raster = raster;
      AttnParams p;
      sta::fill_params(pr, sta::kF32Rows, &p);
      long long worst = -1, outside = 0;
      const long long grid = (long long)p.per_xcd * sta::kXcds;
      for (long long bid = 0; bid < grid; ++bid) {
        const int task = sta::task_of_block(p, (int)bid);
        if (task >= p.n_tasks) continue;
        const Task t = sta::decode_task<sta::kF32Rows>(p, task, 64);
        for (int tid = 0; tid < t.valid_rows; ++tid) {
          const long long tok = raster ? sta::tile_row_raster(p, t.qt, t.qh, t.qw, t.local0 + tid)
                                       : (long long)t.row0 + tid;
          if (tok >= p.S) { ++outside; worst = tok > worst ? tok : worst; }
        }
      }
      printf("float32 forward, padded grid, %s order: %lld query rows map past the %d rows of a "
             "slice (largest row %lld); tile-major rows stay inside its %d rows\n",
             raster ? "raster" : "tile-major", outside, p.S, worst, pr.g.S_pad);
    }
  }
  printf("host model: %lld launches modelled (%lld forwards with a split last round, %lld one-pass "
         "recalls), %lld padded chunk masks from tables, %lld checks, all in bounds\n",
         g_ctx.launches, g_ctx.tail_launches, g_ctx.recall_passes, g_ctx.pad_masks, g_ctx.checks);
  return 0;
}
