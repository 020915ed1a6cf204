// C-ABI entry points of libsta: argument checks, then dispatch to the HIP
// launchers. Nothing here touches the device before every check has passed.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "sta.h"
#include "sta_geometry.h"
#include "sta_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return STA_OK;
}

int elem_size(int dtype) {
  switch (dtype) {
    case STA_BF16: return 2;
    case STA_F32: return 4;
    default: return 0;
  }
}

// Byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a);
  const uintptr_t pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// Checks the volume and tile, fills g. A tile that does not divide the volume
// is allowed: the grid then covers the volume padded up to whole tiles.
int check_volume(int T, int H, int W, const int* tile, sta::Geometry* g) {
  if (!tile) return fail(STA_ERR_INVALID_ARG, "tile is NULL");
  if (T <= 0 || H <= 0 || W <= 0)
    return fail(STA_ERR_INVALID_ARG, "volume (%d,%d,%d) must be positive", T, H, W);
  if (tile[0] <= 0 || tile[1] <= 0 || tile[2] <= 0)
    return fail(STA_ERR_INVALID_ARG, "tile (%d,%d,%d) must be positive", tile[0], tile[1], tile[2]);
  const long long S = (long long)T * H * W;
  g->T = T; g->H = H; g->W = W;
  g->ct = tile[0]; g->ch = tile[1]; g->cw = tile[2];
  g->nt = (T + tile[0] - 1) / tile[0];
  g->nh = (H + tile[1] - 1) / tile[1];
  g->nw = (W + tile[2] - 1) / tile[2];
  const long long tau = (long long)tile[0] * tile[1] * tile[2];
  const long long n_tiles = (long long)g->nt * g->nh * g->nw;
  if (tau * n_tiles > (1LL << 30))
    return fail(STA_ERR_INVALID_ARG, "volume of %lld tokens (%lld with tile padding) is too large", S,
                tau * n_tiles);
  g->n_tiles = (int)n_tiles;
  g->tau = (int)tau;
  g->S = (int)S;
  g->S_pad = (int)(tau * n_tiles);
  g->padded = g->S_pad != g->S;
  return STA_OK;
}

// Checks the per-head windows against the geometry; fills omega (tiles).
int check_windows(const sta::Geometry& g, int heads, const int* window, uint16_t (*omega)[3]) {
  if (!window) return fail(STA_ERR_INVALID_ARG, "window is NULL");
  const int c[3] = {g.ct, g.ch, g.cw};
  const int n[3] = {g.nt, g.nh, g.nw};
  for (int h = 0; h < heads; ++h) {
    for (int a = 0; a < 3; ++a) {
      const int w = window[3 * h + a];
      if (w <= 0 || w % c[a] || w / c[a] > n[a])
        return fail(STA_ERR_INVALID_ARG,
                    "window (%d,%d,%d) of head %d must be a positive multiple of the tile "
                    "(%d,%d,%d) and at most the tile grid (%d,%d,%d)",
                    window[3 * h], window[3 * h + 1], window[3 * h + 2], h, g.ct, g.ch, g.cw,
                    n[0] * c[0], n[1] * c[1], n[2] * c[2]);
      omega[h][a] = (uint16_t)(w / c[a]);
    }
  }
  return STA_OK;
}

// float32 attention kernels take volumes the tile divides only.
int check_f32_padding(const sta::Geometry& g, int dtype) {
  if (g.padded && dtype == STA_F32)
    return fail(STA_ERR_UNSUPPORTED,
                "float32 attention needs a volume the tile divides (volume %dx%dx%d, tile %dx%dx%d)",
                g.T, g.H, g.W, g.ct, g.ch, g.cw);
  return STA_OK;
}

int check_heads(int B, int heads, int head_dim) {
  if (B <= 0 || heads <= 0 || head_dim <= 0)
    return fail(STA_ERR_INVALID_ARG, "B=%d, heads=%d, head_dim=%d must be positive", B, heads,
                head_dim);
  return STA_OK;
}

int launched(int rc) {
  if (rc == 0) return ok();
  if (rc < 0) return rc;  // message already set by the launcher's caller
  return fail(STA_ERR_HIP, "HIP launch failed: %s", sta::hip_error_string(rc));
}

int reorder_common(const void* src, void* dst, int B, int heads, int head_dim, int T, int H,
                   int W, const int* tile, int dtype, void* stream, bool to_tiles) {
  if (!src || !dst) return fail(STA_ERR_INVALID_ARG, "input or output pointer is NULL");
  int rc = check_heads(B, heads, head_dim);
  if (rc) return rc;
  const int es = elem_size(dtype);
  if (!es) return fail(STA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  sta::Geometry g;
  if ((rc = check_volume(T, H, W, tile, &g))) return rc;
  const long long row_bytes = (long long)head_dim * es;
  if (row_bytes % 16)
    return fail(STA_ERR_UNSUPPORTED, "head_dim * element size (%lld bytes) must be a multiple of 16",
                row_bytes);
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return fail(STA_ERR_UNSUPPORTED, "input and output must be 16-byte aligned");
  const long long BH = (long long)B * heads;
  if (BH > (1LL << 24)) return fail(STA_ERR_INVALID_ARG, "B*heads=%lld is too large", BH);
  const size_t raster_bytes = (size_t)BH * g.S * row_bytes;
  const size_t tiled_bytes = (size_t)BH * g.S_pad * row_bytes;
  if (overlaps(src, to_tiles ? raster_bytes : tiled_bytes, dst, to_tiles ? tiled_bytes : raster_bytes))
    return fail(STA_ERR_INVALID_ARG, "input and output overlap");
  return launched(sta::launch_reorder(src, dst, (int)BH, (int)row_bytes, g, to_tiles, stream));
}

int attention_common(sta::AttnProblem& p, void* stream) {
  if (!p.q || !p.k || !p.v || !p.out) return fail(STA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  int rc = check_heads(p.B, p.heads, p.head_dim);
  if (rc) return rc;
  // The work plan keeps per-head tables of STA_MAX_HEADS entries (window,
  // heaviest-first head order), for the dense comparator too.
  if (p.heads > STA_MAX_HEADS)
    return fail(STA_ERR_INVALID_ARG, "heads=%d must be in [1, %d]", p.heads, STA_MAX_HEADS);
  const int es = elem_size(p.dtype);
  if (!es) return fail(STA_ERR_INVALID_ARG, "unknown dtype %d", p.dtype);
  if (!(p.scale > 0.0f) || !isfinite(p.scale))
    return fail(STA_ERR_INVALID_ARG, "scale %g must be finite and positive", (double)p.scale);
  if (p.head_dim != 64 && p.head_dim != 128)
    return fail(STA_ERR_UNSUPPORTED, "head_dim %d: kernels exist for 64 and 128", p.head_dim);
  const uintptr_t any = reinterpret_cast<uintptr_t>(p.q) | reinterpret_cast<uintptr_t>(p.k) |
                        reinterpret_cast<uintptr_t>(p.v) | reinterpret_cast<uintptr_t>(p.out);
  if (any % 16) return fail(STA_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  const long long BH = (long long)p.B * p.heads;
  if (BH > (1LL << 24)) return fail(STA_ERR_INVALID_ARG, "B*heads=%lld is too large", BH);
  const int rows = p.dense || p.raster ? p.g.S : p.g.S_pad;
  const size_t bytes = (size_t)BH * rows * p.head_dim * es;
  const size_t qk_bytes = p.qk_fp8 ? (size_t)BH * rows * p.head_dim : bytes;
  if (overlaps(p.out, bytes, p.q, qk_bytes) || overlaps(p.out, bytes, p.k, qk_bytes) ||
      overlaps(p.out, bytes, p.v, bytes))
    return fail(STA_ERR_INVALID_ARG, "output overlaps an input");
  rc = sta::launch_attention(p, stream);
  if (rc < 0) return fail(rc, "no kernel for dtype %d with head_dim %d", p.dtype, p.head_dim);
  return launched(rc);
}

// Longest list of sta_kv_tiles (transposed = false) or sta_q_tiles (true)
// over heads and tiles, and the longest run along w of such a list in tiles.
void list_extents(const sta::Geometry& g, int heads, const uint16_t (*omega)[3], bool transposed,
                  int* longest, int* longest_w) {
  *longest = 0;
  *longest_w = 0;
  const int n[3] = {g.nt, g.nh, g.nw};
  for (int h = 0; h < heads; ++h) {
    int prod = 1;
    for (int a = 0; a < 3; ++a) {
      int m = omega[h][a];
      if (transposed) {
        m = 0;
        for (int j = 0; j < n[a]; ++j) {
          int lo, hi;
          sta::window_inverse(j, n[a], omega[h][a], &lo, &hi);
          m = hi - lo + 1 > m ? hi - lo + 1 : m;
        }
      }
      prod *= m;
      if (a == 2 && m > *longest_w) *longest_w = m;
    }
    *longest = prod > *longest ? prod : *longest;
  }
}

int tile_lists_common(int* list, int* count, int heads, int T, int H, int W, const int* tile,
                      const int* window, int max_len, bool transposed, void* stream) {
  if (!list || !count) return fail(STA_ERR_INVALID_ARG, "list or count is NULL");
  if (heads <= 0 || heads > STA_MAX_HEADS)
    return fail(STA_ERR_INVALID_ARG, "heads=%d must be in [1, %d]", heads, STA_MAX_HEADS);
  sta::Geometry g;
  int rc = check_volume(T, H, W, tile, &g);
  if (rc) return rc;
  uint16_t omega[STA_MAX_HEADS][3];
  if ((rc = check_windows(g, heads, window, omega))) return rc;
  int need, need_w;
  list_extents(g, heads, omega, transposed, &need, &need_w);
  if (max_len < need)
    return fail(STA_ERR_INVALID_ARG, "list length %d is below the longest list %d", max_len, need);
  const size_t list_bytes = (size_t)heads * g.n_tiles * max_len * sizeof(int);
  const size_t count_bytes = (size_t)heads * g.n_tiles * sizeof(int);
  if (overlaps(list, list_bytes, count, count_bytes))
    return fail(STA_ERR_INVALID_ARG, "list and count overlap");
  if ((long long)heads * g.n_tiles * max_len > (1LL << 31) - 1)
    return fail(STA_ERR_INVALID_ARG, "list is too large");
  return launched(sta::launch_kv_tiles(list, count, heads, g, omega, max_len, transposed, stream));
}

// Raster-order kernels keep the raster offsets of one run in LDS: both the
// window runs (omega_w tiles) and, for the backward, the transposed runs must
// fit.
int check_raster_runs(const sta::Geometry& g, int heads, const uint16_t (*omega)[3], bool backward) {
  int longest, longest_w;
  list_extents(g, heads, omega, false, &longest, &longest_w);
  long long run = (long long)longest_w * g.tau;
  if (backward) {
    list_extents(g, heads, omega, true, &longest, &longest_w);
    const long long trun = (long long)longest_w * g.tau;
    run = trun > run ? trun : run;
  }
  if (run > sta::kMaxRasterRun)
    return fail(STA_ERR_UNSUPPORTED,
                "raster order: a window run has %lld keys (limit %d); reorder to tile-major order "
                "and use the tile-major entry point",
                run, sta::kMaxRasterRun);
  // The kernels address the keys of a run as 32-bit byte offsets from its
  // first key: one tile-row of frames, c_t * H * W tokens of at most 256
  // bytes, must stay below 2 GB.
  const long long span = (long long)g.ct * g.H * g.W * 256;
  if (span >= (1LL << 31))
    return fail(STA_ERR_UNSUPPORTED,
                "raster order: c_t * H * W = %lld tokens exceeds the raster addressing range; "
                "reorder to tile-major order and use the tile-major entry point",
                (long long)g.ct * g.H * g.W);
  return STA_OK;
}

int forward_common(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int heads, int head_dim, int T, int H, int W, const int* tile,
                   const int* window, float scale, int dtype, void* stream, bool raster,
                   bool qk_fp8 = false);

}  // namespace

extern "C" {

int sta_abi_version(void) { return 7; }

const char* sta_last_error(void) { return g_last_error.c_str(); }

int sta_reorder_tiles(const void* x_raster, void* x_tiled, int B, int heads, int head_dim, int T,
                      int H, int W, const int* tile, int dtype, void* stream) {
  return reorder_common(x_raster, x_tiled, B, heads, head_dim, T, H, W, tile, dtype, stream, true);
}

int sta_restore_order(const void* x_tiled, void* x_raster, int B, int heads, int head_dim, int T,
                      int H, int W, const int* tile, int dtype, void* stream) {
  return reorder_common(x_tiled, x_raster, B, heads, head_dim, T, H, W, tile, dtype, stream, false);
}

long long sta_kv_pair_count(int heads, int T, int H, int W, const int* tile, const int* window) {
  if (heads <= 0 || heads > STA_MAX_HEADS)
    return fail(STA_ERR_INVALID_ARG, "heads=%d must be in [1, %d]", heads, STA_MAX_HEADS);
  sta::Geometry g;
  int rc = check_volume(T, H, W, tile, &g);
  if (rc) return rc;
  static thread_local uint16_t omega[STA_MAX_HEADS][3];
  if ((rc = check_windows(g, heads, window, omega))) return rc;
  long long pairs = 0;
  for (int h = 0; h < heads; ++h)
    pairs += (long long)g.n_tiles * omega[h][0] * omega[h][1] * omega[h][2];
  ok();
  return pairs;
}

int sta_tile_list_len(int heads, int T, int H, int W, const int* tile, const int* window,
                      int transposed) {
  if (heads <= 0 || heads > STA_MAX_HEADS)
    return fail(STA_ERR_INVALID_ARG, "heads=%d must be in [1, %d]", heads, STA_MAX_HEADS);
  if (transposed != 0 && transposed != 1)
    return fail(STA_ERR_INVALID_ARG, "transposed=%d must be 0 or 1", transposed);
  sta::Geometry g;
  int rc = check_volume(T, H, W, tile, &g);
  if (rc) return rc;
  static thread_local uint16_t omega[STA_MAX_HEADS][3];
  if ((rc = check_windows(g, heads, window, omega))) return rc;
  int longest, longest_w;
  list_extents(g, heads, omega, transposed != 0, &longest, &longest_w);
  ok();
  return longest;
}

int sta_kv_tiles(int* kv_list, int* kv_count, int heads, int T, int H, int W, const int* tile,
                 const int* window, int max_kv, void* stream) {
  return tile_lists_common(kv_list, kv_count, heads, T, H, W, tile, window, max_kv, false, stream);
}

int sta_q_tiles(int* q_list, int* q_count, int heads, int T, int H, int W, const int* tile,
                const int* window, int max_q, void* stream) {
  return tile_lists_common(q_list, q_count, heads, T, H, W, tile, window, max_q, true, stream);
}

}  // extern "C"

namespace {

int forward_common(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int heads, int head_dim, int T, int H, int W, const int* tile,
                   const int* window, float scale, int dtype, void* stream, bool raster,
                   bool qk_fp8) {
  if (heads <= 0 || heads > STA_MAX_HEADS)
    return fail(STA_ERR_INVALID_ARG, "heads=%d must be in [1, %d]", heads, STA_MAX_HEADS);
  static thread_local sta::AttnProblem p;
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  p.B = B; p.heads = heads; p.head_dim = head_dim; p.dtype = dtype; p.scale = scale;
  p.dense = false;
  p.raster = raster;
  p.lse_only = false;
  p.qk_fp8 = qk_fp8;
  p.n_cand = 0;
  int rc = check_volume(T, H, W, tile, &p.g);
  if (rc) return rc;
  if ((rc = check_windows(p.g, heads, window, p.omega))) return rc;
  if ((rc = check_f32_padding(p.g, dtype))) return rc;
  if (raster && (rc = check_raster_runs(p.g, heads, p.omega, false))) return rc;
  if (lse) {
    if (reinterpret_cast<uintptr_t>(lse) % 4) return fail(STA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
    const int es = elem_size(dtype);
    const int rows = raster ? p.g.S : p.g.S_pad;
    const size_t bytes = (size_t)B * heads * rows * (es ? es : 1) * head_dim;
    const size_t qk_bytes = qk_fp8 ? (size_t)B * heads * rows * head_dim : bytes;
    const size_t lbytes = (size_t)B * heads * rows * sizeof(float);
    if (overlaps(lse, lbytes, q, qk_bytes) || overlaps(lse, lbytes, k, qk_bytes) ||
        overlaps(lse, lbytes, v, bytes) || overlaps(lse, lbytes, out, bytes))
      return fail(STA_ERR_INVALID_ARG, "lse overlaps a tensor");
  }
  return attention_common(p, stream);
}

// use_scratch: D goes to the library's static device scratch (delta is
// ignored); the problem must fit it.
int backward_common(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    float* delta, int B, int heads, int head_dim, int T, int H, int W,
                    const int* tile, const int* window, float scale, int dtype, int order,
                    void* stream, bool use_scratch = false) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || (!delta && !use_scratch))
    return fail(STA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (order != STA_TILE_MAJOR && order != STA_RASTER)
    return fail(STA_ERR_INVALID_ARG, "unknown token order %d", order);
  if (heads <= 0 || heads > STA_MAX_HEADS)
    return fail(STA_ERR_INVALID_ARG, "heads=%d must be in [1, %d]", heads, STA_MAX_HEADS);
  int rc = check_heads(B, heads, head_dim);
  if (rc) return rc;
  const int es = elem_size(dtype);
  if (!es) return fail(STA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(STA_ERR_INVALID_ARG, "scale %g must be finite and positive", (double)scale);
  if (head_dim != 64 && head_dim != 128)
    return fail(STA_ERR_UNSUPPORTED, "head_dim %d: kernels exist for 64 and 128", head_dim);
  static thread_local sta::BwdProblem pb;
  sta::AttnProblem& p = pb.attn;
  p.q = q; p.k = k; p.v = v; p.out = const_cast<void*>(out); p.lse = nullptr;
  p.B = B; p.heads = heads; p.head_dim = head_dim; p.dtype = dtype; p.scale = scale;
  p.dense = false;
  p.raster = order == STA_RASTER;
  p.lse_only = false;
  p.qk_fp8 = false;
  p.n_cand = 0;
  if ((rc = check_volume(T, H, W, tile, &p.g))) return rc;
  if ((rc = check_windows(p.g, heads, window, p.omega))) return rc;
  if ((rc = check_f32_padding(p.g, dtype))) return rc;
  if (p.raster && (rc = check_raster_runs(p.g, heads, p.omega, true))) return rc;
  const uintptr_t any16 = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out) |
                          reinterpret_cast<uintptr_t>(dout) | reinterpret_cast<uintptr_t>(dq) |
                          reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv);
  if (any16 % 16) return fail(STA_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(delta)) % 4)
    return fail(STA_ERR_INVALID_ARG, "lse and delta must be 4-byte aligned");
  const long long BH = (long long)B * heads;
  if (BH > (1LL << 24)) return fail(STA_ERR_INVALID_ARG, "B*heads=%lld is too large", BH);
  const int rows = p.raster ? p.g.S : p.g.S_pad;
  if (use_scratch && BH * rows > sta::kNoAllocScratchFloats)
    return fail(STA_ERR_INVALID_ARG,
                "B*heads*rows = %lld exceeds the %lld rows of the allocation-free scratch; "
                "use sta_backward with a caller-owned delta workspace",
                BH * rows, sta::kNoAllocScratchFloats);
  const size_t tb = (size_t)BH * rows * head_dim * es;
  const size_t rb = (size_t)BH * rows * sizeof(float);
  const void* ins[6] = {q, k, v, out, dout, lse};
  const size_t in_bytes[6] = {tb, tb, tb, tb, tb, rb};
  const void* outs[4] = {dq, dk, dv, delta};
  const size_t out_bytes[4] = {tb, tb, tb, rb};
  const int n_outs = use_scratch ? 3 : 4;   // the library's own scratch overlaps nothing
  for (int i = 0; i < n_outs; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j]))
        return fail(STA_ERR_INVALID_ARG, "an output or the delta workspace overlaps an input");
    for (int j = i + 1; j < n_outs; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j]))
        return fail(STA_ERR_INVALID_ARG, "outputs overlap each other or the delta workspace");
  }
  if (use_scratch) {   // every check has passed: look up this device's scratch
    const int e = sta::noalloc_scratch(&delta);
    if (e) return fail(STA_ERR_HIP, "device scratch lookup failed: %s", sta::hip_error_string(e));
  }
  pb.dout = dout; pb.lse = lse; pb.delta = delta;
  pb.dq = dq; pb.dk = dk; pb.dv = dv;
  rc = sta::launch_backward(pb, stream);
  if (rc < 0) return fail(rc, "no kernel for dtype %d with head_dim %d", dtype, head_dim);
  return launched(rc);
}

}  // namespace

extern "C" {

int sta_forward(const void* q, const void* k, const void* v, void* out, int B, int heads,
                int head_dim, int T, int H, int W, const int* tile, const int* window, float scale,
                int dtype, void* stream) {
  return forward_common(q, k, v, out, nullptr, B, heads, head_dim, T, H, W, tile, window, scale,
                        dtype, stream, false);
}

int sta_forward_raster(const void* q, const void* k, const void* v, void* out, int B, int heads,
                       int head_dim, int T, int H, int W, const int* tile, const int* window,
                       float scale, int dtype, void* stream) {
  return forward_common(q, k, v, out, nullptr, B, heads, head_dim, T, H, W, tile, window, scale,
                        dtype, stream, true);
}

int sta_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                    int heads, int head_dim, int T, int H, int W, const int* tile,
                    const int* window, float scale, int dtype, int order, void* stream) {
  if (!lse) return fail(STA_ERR_INVALID_ARG, "lse is NULL");
  if (order != STA_TILE_MAJOR && order != STA_RASTER)
    return fail(STA_ERR_INVALID_ARG, "unknown token order %d", order);
  return forward_common(q, k, v, out, lse, B, heads, head_dim, T, H, W, tile, window, scale,
                        dtype, stream, order == STA_RASTER);
}

namespace {

int forward_fp8_common(const void* q8, const void* k8, const void* v, void* out, float* lse, int B,
                       int heads, int head_dim, int T, int H, int W, const int* tile,
                       const int* window, float scale, float q_descale, float k_descale, int order,
                       void* stream) {
  if (order != STA_TILE_MAJOR && order != STA_RASTER)
    return fail(STA_ERR_INVALID_ARG, "unknown token order %d", order);
  if (!(q_descale > 0.0f) || !isfinite(q_descale) || !(k_descale > 0.0f) || !isfinite(k_descale))
    return fail(STA_ERR_INVALID_ARG, "descales %g, %g must be finite and positive",
                (double)q_descale, (double)k_descale);
  if (head_dim != 128)
    return fail(STA_ERR_UNSUPPORTED, "head_dim %d: the fp8 kernels need 128", head_dim);
  const float folded = scale * q_descale * k_descale;
  if (!(scale > 0.0f) || !isfinite(scale) || !(folded > 0.0f) || !isfinite(folded))
    return fail(STA_ERR_INVALID_ARG, "scale %g times the descales must be finite and positive",
                (double)scale);
  return forward_common(q8, k8, v, out, lse, B, heads, head_dim, T, H, W, tile, window, folded,
                        STA_BF16, stream, order == STA_RASTER, true);
}

}  // namespace

int sta_forward_fp8(const void* q8, const void* k8, const void* v, void* out, int B, int heads,
                    int head_dim, int T, int H, int W, const int* tile, const int* window,
                    float scale, float q_descale, float k_descale, int order, void* stream) {
  return forward_fp8_common(q8, k8, v, out, nullptr, B, heads, head_dim, T, H, W, tile, window,
                            scale, q_descale, k_descale, order, stream);
}

int sta_forward_fp8_lse(const void* q8, const void* k8, const void* v, void* out, float* lse, int B,
                        int heads, int head_dim, int T, int H, int W, const int* tile,
                        const int* window, float scale, float q_descale, float k_descale,
                        int order, void* stream) {
  if (!lse) return fail(STA_ERR_INVALID_ARG, "lse is NULL");
  return forward_fp8_common(q8, k8, v, out, lse, B, heads, head_dim, T, H, W, tile, window, scale,
                            q_descale, k_descale, order, stream);
}

int sta_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int heads,
                 int head_dim, int T, int H, int W, const int* tile, const int* window,
                 float scale, int dtype, int order, void* stream) {
  return backward_common(q, k, v, out, dout, lse, dq, dk, dv, delta, B, heads, head_dim, T, H, W,
                         tile, window, scale, dtype, order, stream);
}

int sta_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int heads, int head_dim, int T, int H, int W, const int* tile,
                         const int* window, float scale, int dtype, int order, void* stream) {
  return backward_common(q, k, v, out, dout, lse, dq, dk, dv, nullptr, B, heads, head_dim, T, H, W,
                         tile, window, scale, dtype, order, stream, true);
}

namespace {

// Window recall for bf16 / float32 q, k, or fp8 codes (qk_fp8: dtype is
// STA_BF16, scale already carries the descales).
int recall_common(const void* q, const void* k, float* recall, float* workspace, int B, int heads,
                  int head_dim, int T, int H, int W, const int* tile, const int* candidates,
                  int n_candidates, float scale, int dtype, int order, void* stream, bool qk_fp8) {
  if (!q || !k || !recall || !workspace || !candidates)
    return fail(STA_ERR_INVALID_ARG, "a pointer is NULL");
  if (n_candidates <= 0) return fail(STA_ERR_INVALID_ARG, "n_candidates=%d must be positive", n_candidates);
  if (order != STA_TILE_MAJOR && order != STA_RASTER)
    return fail(STA_ERR_INVALID_ARG, "unknown token order %d", order);
  if (heads <= 0 || heads > STA_MAX_HEADS)
    return fail(STA_ERR_INVALID_ARG, "heads=%d must be in [1, %d]", heads, STA_MAX_HEADS);
  int rc = check_heads(B, heads, head_dim);
  if (rc) return rc;
  const int es = elem_size(dtype);
  if (!es) return fail(STA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(STA_ERR_INVALID_ARG, "scale %g must be finite and positive", (double)scale);
  if (head_dim != 64 && head_dim != 128)
    return fail(STA_ERR_UNSUPPORTED, "head_dim %d: kernels exist for 64 and 128", head_dim);
  static thread_local sta::AttnProblem dense, win;
  if ((rc = check_volume(T, H, W, tile, &win.g))) return rc;
  if ((rc = check_f32_padding(win.g, dtype))) return rc;
  if (win.g.padded && order != STA_RASTER)
    return fail(STA_ERR_UNSUPPORTED,
                "window recall on a volume the tile does not divide needs raster order (the "
                "full-attention pass would see the padding rows of a tile-major tensor)");
  // every candidate is a valid window (checked as one head each)
  static thread_local uint16_t om[STA_MAX_HEADS][3];
  for (int c = 0; c < n_candidates; ++c)
    if ((rc = check_windows(win.g, 1, candidates + 3 * c, om))) return rc;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k)) % 16)
    return fail(STA_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(recall) | reinterpret_cast<uintptr_t>(workspace)) % 4)
    return fail(STA_ERR_INVALID_ARG, "recall and workspace must be 4-byte aligned");
  const long long BH = (long long)B * heads;
  if (BH > (1LL << 24)) return fail(STA_ERR_INVALID_ARG, "B*heads=%lld is too large", BH);
  const size_t tb = (size_t)BH * win.g.S * head_dim * (qk_fp8 ? 1 : es);
  const size_t wb = (size_t)(n_candidates + 1) * BH * win.g.S * sizeof(float);
  const size_t rb = (size_t)BH * n_candidates * sizeof(float);
  if (overlaps(workspace, wb, q, tb) || overlaps(workspace, wb, k, tb) ||
      overlaps(recall, rb, q, tb) || overlaps(recall, rb, k, tb) || overlaps(recall, rb, workspace, wb))
    return fail(STA_ERR_INVALID_ARG, "recall or workspace overlaps an input or each other");
  float* lse_full = workspace;
  const size_t slot = (size_t)BH * win.g.S;
  // One pass per group of up to kMaxRecallCand candidates when the kernels
  // allow it: STA with the whole volume as every head's window (full
  // attention) that also sums, per candidate, the probabilities of the keys
  // the candidate's window holds. Every pass writes the same full lse.
  if (!win.g.padded) {
    static thread_local sta::AttnProblem one;
    one.q = q; one.k = k; one.v = k; one.out = nullptr; one.lse = lse_full;
    one.B = B; one.heads = heads; one.head_dim = head_dim; one.dtype = dtype; one.scale = scale;
    one.dense = false; one.raster = order == STA_RASTER; one.lse_only = true; one.qk_fp8 = qk_fp8;
    one.g = win.g;
    for (int h = 0; h < heads; ++h) {
      one.omega[h][0] = (uint16_t)win.g.nt;
      one.omega[h][1] = (uint16_t)win.g.nh;
      one.omega[h][2] = (uint16_t)win.g.nw;
    }
    one.cand_stride = (long long)slot;
    bool done = true;
    for (int c0 = 0; c0 < n_candidates && done; c0 += sta::kMaxRecallCand) {
      one.n_cand = n_candidates - c0 < sta::kMaxRecallCand ? n_candidates - c0 : sta::kMaxRecallCand;
      one.lse_cand = workspace + (c0 + 1) * slot;
      for (int c = 0; c < one.n_cand; ++c) {
        one.cand_omega[c][0] = (uint16_t)(candidates[3 * (c0 + c)] / win.g.ct);
        one.cand_omega[c][1] = (uint16_t)(candidates[3 * (c0 + c) + 1] / win.g.ch);
        one.cand_omega[c][2] = (uint16_t)(candidates[3 * (c0 + c) + 2] / win.g.cw);
      }
      rc = sta::launch_attention(one, stream);
      if (rc > 0) return launched(rc);
      done = rc == 0;   // no one-pass kernel for this problem: the first group falls back
    }
    if (done) {
      for (int c = 0; c < n_candidates; ++c) {
        rc = sta::launch_recall_reduce(lse_full, workspace + (c + 1) * slot, recall, (int)BH, win.g.S,
                                       n_candidates, c, stream);
        if (rc) return launched(rc);
      }
      return ok();
    }
    // no one-pass kernel for this problem: one pass per candidate below
  }
  // full-attention lse (token order does not matter for all-keys attention)
  dense.q = q; dense.k = k; dense.v = k; dense.out = nullptr; dense.lse = lse_full;
  dense.B = B; dense.heads = heads; dense.head_dim = head_dim; dense.dtype = dtype; dense.scale = scale;
  dense.dense = true; dense.raster = false; dense.lse_only = true; dense.qk_fp8 = qk_fp8;
  dense.n_cand = 0;
  memset(&dense.g, 0, sizeof(dense.g));
  dense.g.S = win.g.S;
  rc = sta::launch_attention(dense, stream);
  if (rc) return rc < 0 ? fail(rc, "no kernel for dtype %d with head_dim %d", dtype, head_dim) : launched(rc);
  win.q = q; win.k = k; win.v = k; win.out = nullptr;
  win.B = B; win.heads = heads; win.head_dim = head_dim; win.dtype = dtype; win.scale = scale;
  win.dense = false; win.raster = order == STA_RASTER; win.lse_only = true; win.qk_fp8 = qk_fp8;
  win.n_cand = 0;
  for (int c = 0; c < n_candidates; ++c) {
    for (int h = 0; h < heads; ++h) {
      win.omega[h][0] = (uint16_t)(candidates[3 * c] / win.g.ct);
      win.omega[h][1] = (uint16_t)(candidates[3 * c + 1] / win.g.ch);
      win.omega[h][2] = (uint16_t)(candidates[3 * c + 2] / win.g.cw);
    }
    if (win.raster && (rc = check_raster_runs(win.g, heads, win.omega, false))) return rc;
    win.lse = workspace + (c + 1) * slot;   // candidate c's row lse
    rc = sta::launch_attention(win, stream);
    if (rc) return rc < 0 ? fail(rc, "no kernel for dtype %d with head_dim %d", dtype, head_dim) : launched(rc);
    rc = sta::launch_recall_reduce(lse_full, win.lse, recall, (int)BH, win.g.S, n_candidates, c, stream);
    if (rc) return launched(rc);
  }
  return ok();
}

}  // namespace

int sta_window_recall(const void* q, const void* k, float* recall, float* workspace, int B,
                      int heads, int head_dim, int T, int H, int W, const int* tile,
                      const int* candidates, int n_candidates, float scale, int dtype, int order,
                      void* stream) {
  return recall_common(q, k, recall, workspace, B, heads, head_dim, T, H, W, tile, candidates,
                       n_candidates, scale, dtype, order, stream, false);
}

int sta_window_recall_fp8(const void* q8, const void* k8, float* recall, float* workspace, int B,
                          int heads, int head_dim, int T, int H, int W, const int* tile,
                          const int* candidates, int n_candidates, float scale, float q_descale,
                          float k_descale, int order, void* stream) {
  if (!(q_descale > 0.0f) || !isfinite(q_descale) || !(k_descale > 0.0f) || !isfinite(k_descale))
    return fail(STA_ERR_INVALID_ARG, "descales %g, %g must be finite and positive",
                (double)q_descale, (double)k_descale);
  if (head_dim != 128)
    return fail(STA_ERR_UNSUPPORTED, "head_dim %d: the fp8 kernels need 128", head_dim);
  const float folded = scale * q_descale * k_descale;
  if (!(scale > 0.0f) || !isfinite(scale) || !(folded > 0.0f) || !isfinite(folded))
    return fail(STA_ERR_INVALID_ARG, "scale %g times the descales must be finite and positive",
                (double)scale);
  return recall_common(q8, k8, recall, workspace, B, heads, head_dim, T, H, W, tile, candidates,
                       n_candidates, folded, STA_BF16, order, stream, true);
}

int sta_full_attention(const void* q, const void* k, const void* v, void* out, int B, int heads,
                       int head_dim, int S, float scale, int dtype, void* stream) {
  if (S <= 0 || S > (1 << 30)) return fail(STA_ERR_INVALID_ARG, "S=%d must be in [1, 2^30]", S);
  static thread_local sta::AttnProblem p;
  memset(&p.g, 0, sizeof(p.g));
  p.raster = false;
  p.lse_only = false;
  p.qk_fp8 = false;
  p.n_cand = 0;
  p.lse = nullptr;
  p.q = q; p.k = k; p.v = v; p.out = out;
  p.B = B; p.heads = heads; p.head_dim = head_dim; p.dtype = dtype; p.scale = scale;
  p.dense = true;
  p.g.S = S;
  return attention_common(p, stream);
}

}  // extern "C"
