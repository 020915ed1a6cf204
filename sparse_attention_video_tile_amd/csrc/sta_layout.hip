// Token-order and tile-list kernels of libsta (gfx950).
//
// reorder_kernel: raster <-> tile-major permutation of the token axis. A
// wavefront moves one tile of one (batch, head): it walks the tile's
// contiguous tile-major range in 1 KB steps (16 bytes per lane). Each 16-byte
// chunk lies in one run, the c_w tokens that share (t, y), which is also
// contiguous in raster order, so both sides are coalesced. Sixteen chunks per
// lane are loaded before any is stored, to keep enough bytes in flight, with
// non-temporal loads and stores (the data is touched once): 96-99 % of the
// bandwidth of a plain device copy of the same tensor, against 92 % with
// eight cached chunks per lane.
//
// kv_tiles_kernel: one thread per (head, tile, list slot) writes the slot's
// tile of the window box (or of the transposed window), in (t, h, w)
// lexicographic order, which is ascending tile index.
#include <hip/hip_runtime.h>

#include "sta_kernels.h"

namespace sta {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReorderThreads = 256;
constexpr int kUnroll = 16;  // 16-byte chunks per lane whose loads are in flight together

// Unsigned division by a divisor fixed for the whole launch, as a multiply
// and shift (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): for n < 2^31, n / d = (umulhi(n, m) + n) >> s with
// s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1.
struct FastDiv {
  uint32_t d, m, s;
  static FastDiv make(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.s = 0;
    while ((1ull << f.s) < d) ++f.s;
    f.m = (uint32_t)(((1ull << 32) * ((1ull << f.s) - d)) / d + 1);
    return f;
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (__umulhi(n, m) + n) >> s;
  }
};

struct ReorderParams {
  const u32x4* src;
  u32x4* dst;
  long long tasks;   // BH * n_tiles: one (head, tile) per wavefront
  int tile_chunks;   // tau * row_chunks: 16-byte chunks in one tile
  int row_chunks;    // 16-byte chunks per token row
  int S, S_pad, T, H, W;  // raster rows, tile-major rows, volume
  int ct, ch, cw, nh, nw, n_tiles, tau;
  FastDiv run_div;   // by row_chunks * cw: chunk -> run
  FastDiv ch_div;    // by ch: run -> (lt, lh)
  int run_chunks;
  int to_tiles;
};

// One wavefront moves one tile of one (batch, head). Chunk e of the tile in
// tile-major order (contiguous) belongs to run e / run_chunks; a run is the
// cw tokens that share (t, y), contiguous in raster order too. A tile that
// reaches past the volume (tile grid padded up to whole tiles) takes a slower
// loop that checks every row: padded rows are written as zeros in tile-major
// order and skipped when restoring.
__global__ void __launch_bounds__(kReorderThreads) reorder_kernel(const ReorderParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long task = (long long)blockIdx.x * (kReorderThreads / 64) + wave;
  if (task >= p.tasks) return;
  const int tile = (int)(task % p.n_tiles);
  const long long bh = task / p.n_tiles;
  const int iw = tile % p.nw;
  const int ih = (tile / p.nw) % p.nh;
  const int it = tile / (p.nw * p.nh);
  const long long raster_head = bh * p.S * (long long)p.row_chunks;
  const long long tiled_head = bh * p.S_pad * (long long)p.row_chunks;
  // Raster chunk offset of the tile's first run, and per-(lt, lh) strides.
  const long long raster0 =
      raster_head + (((long long)it * p.ct * p.H + ih * p.ch) * p.W + iw * p.cw) * p.row_chunks;
  const long long tiled0 = tiled_head + (long long)tile * p.tile_chunks;
  const long long lt_stride = (long long)p.H * p.W * p.row_chunks;
  const long long lh_stride = (long long)p.W * p.row_chunks;

  auto raster_of = [&](int e) -> long long {
    const uint32_t run = p.run_div.div((uint32_t)e);
    const int c = e - (int)run * p.run_chunks;
    const uint32_t lt = p.ch_div.div(run);
    const int lh = (int)run - (int)lt * p.ch;
    return raster0 + lt * lt_stride + lh * lh_stride + c;
  };

  const u32x4* __restrict__ src = p.src;
  u32x4* __restrict__ dst = p.dst;
  if ((it + 1) * p.ct > p.T || (ih + 1) * p.ch > p.H || (iw + 1) * p.cw > p.W) {
    // edge tile: check each row against the volume
    for (int e = lane; e < p.tile_chunks; e += 64) {
      const uint32_t run = p.run_div.div((uint32_t)e);
      const int c = e - (int)run * p.run_chunks;
      const uint32_t lt = p.ch_div.div(run);
      const int lh = (int)run - (int)lt * p.ch;
      const int lw = c / p.row_chunks;
      const bool real = it * p.ct + (int)lt < p.T && ih * p.ch + lh < p.H && iw * p.cw + lw < p.W;
      if (p.to_tiles) {
        dst[tiled0 + e] = real ? src[raster0 + lt * lt_stride + lh * lh_stride + c] : u32x4{0u, 0u, 0u, 0u};
      } else if (real) {
        dst[raster0 + lt * lt_stride + lh * lh_stride + c] = src[tiled0 + e];
      }
    }
    return;
  }
  int e0 = 0;
  for (; e0 + 64 * kUnroll <= p.tile_chunks; e0 += 64 * kUnroll) {
    u32x4 buf[kUnroll];
    long long soff[kUnroll], doff[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = e0 + 64 * u + lane;
      const long long r = raster_of(e);
      soff[u] = p.to_tiles ? r : tiled0 + e;
      doff[u] = p.to_tiles ? tiled0 + e : r;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) buf[u] = __builtin_nontemporal_load(src + soff[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(buf[u], dst + doff[u]);
  }
  for (int e = e0 + lane; e < p.tile_chunks; e += 64) {
    const long long r = raster_of(e);
    const long long so = p.to_tiles ? r : tiled0 + e;
    const long long d = p.to_tiles ? tiled0 + e : r;
    dst[d] = src[so];
  }
}

struct KvTilesParams {
  int* kv_list;
  int* kv_count;
  long long total;  // heads * n_tiles * max_kv
  int max_kv, n_tiles, nt, nh, nw;
  int transposed;   // 0: key tiles of each query tile's window; 1: query tiles whose window holds each key tile
  uint16_t omega[STA_MAX_HEADS][3];
};

// One thread per (head, tile, list slot). Per axis the listed tiles form an
// interval [lo, hi] (the window, or its transpose); slots enumerate the box in
// (t, h, w) lexicographic order, which is ascending tile index.
__global__ void __launch_bounds__(256) kv_tiles_kernel(const KvTilesParams p) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.total) return;
  const int slot = (int)(idx % p.max_kv);
  const long long rest = idx / p.max_kv;
  const int tile = (int)(rest % p.n_tiles);
  const int h = (int)(rest / p.n_tiles);
  const int tw = tile % p.nw;
  const int th = (tile / p.nw) % p.nh;
  const int tt = tile / (p.nw * p.nh);
  int lo[3], len[3];
  const int c[3] = {tt, th, tw};
  const int n[3] = {p.nt, p.nh, p.nw};
  for (int a = 0; a < 3; ++a) {
    if (p.transposed) {
      int hi;
      window_inverse(c[a], n[a], p.omega[h][a], &lo[a], &hi);
      len[a] = hi - lo[a] + 1;
    } else {
      lo[a] = window_start(c[a], n[a], p.omega[h][a]);
      len[a] = p.omega[h][a];
    }
  }
  const int count = len[0] * len[1] * len[2];
  int value = -1;
  if (slot < count) {
    const int a = slot / (len[1] * len[2]);
    const int b = (slot / len[2]) % len[1];
    const int d = slot % len[2];
    value = ((lo[0] + a) * p.nh + (lo[1] + b)) * p.nw + (lo[2] + d);
  }
  p.kv_list[idx] = value;
  if (slot == 0) p.kv_count[rest] = count;
}

}  // namespace

int launch_reorder(const void* src, void* dst, int BH, int row_bytes, const Geometry& g,
                   bool to_tiles, void* stream) {
  ReorderParams p;
  p.src = static_cast<const u32x4*>(src);
  p.dst = static_cast<u32x4*>(dst);
  p.tasks = (long long)BH * g.n_tiles;
  p.row_chunks = row_bytes / 16;
  p.tile_chunks = g.tau * p.row_chunks;
  p.run_chunks = p.row_chunks * g.cw;
  p.S = g.S; p.S_pad = g.S_pad; p.T = g.T; p.H = g.H; p.W = g.W;
  p.ct = g.ct; p.ch = g.ch; p.cw = g.cw; p.nh = g.nh; p.nw = g.nw;
  p.n_tiles = g.n_tiles; p.tau = g.tau;
  p.run_div = FastDiv::make((uint32_t)p.run_chunks);
  p.ch_div = FastDiv::make((uint32_t)g.ch);
  p.to_tiles = to_tiles ? 1 : 0;
  if ((long long)p.tile_chunks >= (1LL << 31)) return (int)hipErrorInvalidValue;
  const long long waves_per_block = kReorderThreads / 64;
  const long long blocks = (p.tasks + waves_per_block - 1) / waves_per_block;
  if (blocks > 0x7fffffffLL) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(reorder_kernel, dim3((unsigned)blocks), dim3(kReorderThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

int launch_kv_tiles(int* kv_list, int* kv_count, int heads, const Geometry& g,
                    const uint16_t (*omega)[3], int max_kv, bool transposed, void* stream) {
  KvTilesParams p;
  p.transposed = transposed ? 1 : 0;
  p.kv_list = kv_list;
  p.kv_count = kv_count;
  p.total = (long long)heads * g.n_tiles * max_kv;
  p.max_kv = max_kv;
  p.n_tiles = g.n_tiles; p.nt = g.nt; p.nh = g.nh; p.nw = g.nw;
  for (int h = 0; h < heads; ++h)
    for (int a = 0; a < 3; ++a) p.omega[h][a] = omega[h][a];
  const long long blocks = (p.total + 255) / 256;
  hipLaunchKernelGGL(kv_tiles_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

const char* hip_error_string(int code) { return hipGetErrorString(static_cast<hipError_t>(code)); }

}  // namespace sta
