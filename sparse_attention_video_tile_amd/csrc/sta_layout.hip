// Token-order and tile-list kernels of libsta (gfx950).
//
// reorder_kernel: raster <-> tile-major permutation of the token axis. A
// wavefront moves one tile of one (batch, head). The tile is c_t * c_h runs;
// a run is the c_w tokens that share (t, y), contiguous in both orders
// (c_w * row_bytes bytes), so each is copied with 16-byte loads and stores that
// are coalesced on both sides. Loads of several runs are issued before their
// stores to keep enough bytes in flight for HBM.
//
// kv_tiles_kernel: one thread per (head, query tile, list slot) writes the
// slot's key tile, walking the window box in (t, h, w) lexicographic order,
// which is ascending tile index.
#include <hip/hip_runtime.h>

#include "sta_kernels.h"

namespace sta {
namespace {

constexpr int kReorderThreads = 256;
constexpr int kRunsInFlight = 4;   // runs whose loads are issued before their stores
constexpr int kChunksPerLane = 2;  // 16-byte chunks per lane per run and pass

struct ReorderParams {
  const uint4* __restrict__ src;
  uint4* __restrict__ dst;
  long long tasks;  // BH * n_tiles: one (head, tile) per wavefront
  int row_chunks;   // 16-byte chunks per token row
  int run_chunks;   // row_chunks * cw: one contiguous run
  int S, H, W;
  int ct, ch, cw, nh, nw, n_tiles, tau;
  int to_tiles;
};

// One wavefront moves one tile of one (batch, head): ct * ch runs of cw rows.
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
  const long long head_row = bh * p.S;
  const long long raster0 = head_row + ((long long)it * p.ct * p.H + ih * p.ch) * p.W + iw * p.cw;
  const long long tiled0 = head_row + (long long)tile * p.tau;
  const int runs = p.ct * p.ch;
  for (int c0 = 0; c0 < p.run_chunks; c0 += 64 * kChunksPerLane) {
    for (int r0 = 0; r0 < runs; r0 += kRunsInFlight) {
      uint4 buf[kRunsInFlight][kChunksPerLane];
      long long dst_off[kRunsInFlight];
#pragma unroll
      for (int i = 0; i < kRunsInFlight; ++i) {
        const int run = r0 + i;
        const int lt = run / p.ch, lh = run % p.ch;
        const long long raster_row = raster0 + ((long long)lt * p.H + lh) * p.W;
        const long long tiled_row = tiled0 + (long long)run * p.cw;
        const long long src_row = p.to_tiles ? raster_row : tiled_row;
        dst_off[i] = (p.to_tiles ? tiled_row : raster_row) * p.row_chunks;
#pragma unroll
        for (int j = 0; j < kChunksPerLane; ++j) {
          const int c = c0 + lane + 64 * j;
          if (run < runs && c < p.run_chunks) buf[i][j] = p.src[src_row * p.row_chunks + c];
        }
      }
#pragma unroll
      for (int i = 0; i < kRunsInFlight; ++i) {
#pragma unroll
        for (int j = 0; j < kChunksPerLane; ++j) {
          const int c = c0 + lane + 64 * j;
          if (r0 + i < runs && c < p.run_chunks) p.dst[dst_off[i] + c] = buf[i][j];
        }
      }
    }
  }
}

struct KvTilesParams {
  int* kv_list;
  int* kv_count;
  long long total;  // heads * n_tiles * max_kv
  int max_kv, n_tiles, nt, nh, nw;
  uint16_t omega[STA_MAX_HEADS][3];
};

__global__ void __launch_bounds__(256) kv_tiles_kernel(const KvTilesParams p) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.total) return;
  const int slot = (int)(idx % p.max_kv);
  const long long rest = idx / p.max_kv;
  const int qtile = (int)(rest % p.n_tiles);
  const int h = (int)(rest / p.n_tiles);
  const int ot = p.omega[h][0], oh = p.omega[h][1], ow = p.omega[h][2];
  const int qw = qtile % p.nw;
  const int qh = (qtile / p.nw) % p.nh;
  const int qt = qtile / (p.nw * p.nh);
  const int st = window_start(qt, p.nt, ot);
  const int sh = window_start(qh, p.nh, oh);
  const int sw = window_start(qw, p.nw, ow);
  const int count = ot * oh * ow;
  int value = -1;
  if (slot < count) {
    const int a = slot / (oh * ow);
    const int b = (slot / ow) % oh;
    const int c = slot % ow;
    value = ((st + a) * p.nh + (sh + b)) * p.nw + (sw + c);
  }
  p.kv_list[idx] = value;
  if (slot == 0) p.kv_count[rest] = count;
}

}  // namespace

int launch_reorder(const void* src, void* dst, int BH, int row_bytes, const Geometry& g,
                   bool to_tiles, void* stream) {
  ReorderParams p;
  p.src = static_cast<const uint4*>(src);
  p.dst = static_cast<uint4*>(dst);
  p.tasks = (long long)BH * g.n_tiles;
  p.row_chunks = row_bytes / 16;
  p.run_chunks = p.row_chunks * g.cw;
  p.S = g.S; p.H = g.H; p.W = g.W;
  p.ct = g.ct; p.ch = g.ch; p.cw = g.cw; p.nh = g.nh; p.nw = g.nw;
  p.n_tiles = g.n_tiles; p.tau = g.tau;
  p.to_tiles = to_tiles ? 1 : 0;
  const long long waves_per_block = kReorderThreads / 64;
  const long long blocks = (p.tasks + waves_per_block - 1) / waves_per_block;
  hipLaunchKernelGGL(reorder_kernel, dim3((unsigned)blocks), dim3(kReorderThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

int launch_kv_tiles(int* kv_list, int* kv_count, int heads, const Geometry& g,
                    const uint16_t (*omega)[3], int max_kv, void* stream) {
  KvTilesParams p;
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
