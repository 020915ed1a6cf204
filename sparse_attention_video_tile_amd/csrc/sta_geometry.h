// Integer geometry of Sliding Tile Attention, shared by the host checks and
// the HIP kernels of libsta.
//
// A (T, H, W) token volume is cut into (c_t, c_h, c_w) tiles; a head's window
// is a whole number of tiles per axis. The window keeps its size at the border
// of the volume: its start along an axis is the query tile minus half the
// window (rounded down), clamped into [0, n - omega].
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define STA_HD __host__ __device__ __forceinline__
#else
#define STA_HD inline
#endif

namespace sta {

// First key tile of the window along one axis of n tiles, for query tile q
// and a window of omega tiles (1 <= omega <= n).
STA_HD int window_start(int q, int n, int omega) {
  int s = q - omega / 2;
  s = s < 0 ? 0 : s;
  const int hi = n - omega;
  return s > hi ? hi : s;
}

// Query tiles along one axis whose window holds key tile j: the interval
// [*lo, *hi]. window_start is nondecreasing in q, so the set is an interval.
// start(q) <= j holds for every q once j >= n - omega, else exactly for
// q <= j + omega/2; start(q) >= j - omega + 1 holds for every q when that
// bound is <= 0, else exactly for q >= j - omega + 1 + omega/2.
STA_HD void window_inverse(int j, int n, int omega, int* lo, int* hi) {
  const int half = omega / 2;
  *hi = j >= n - omega ? n - 1 : j + half;
  const int a = j - omega + 1;
  *lo = a <= 0 ? 0 : a + half;
}

// A volume the tile does not divide is covered by ceil(extent / c) tiles per
// axis, as if padded up to whole tiles; positions past the volume are not
// tokens. Tile-major tensors hold n_tiles * tau rows (S_pad), raster tensors
// S = T * H * W rows.
struct Geometry {
  int T, H, W;     // tokens per axis
  int ct, ch, cw;  // tile size in tokens
  int nt, nh, nw;  // tiles per axis (ceil(extent / c))
  int n_tiles;     // nt * nh * nw
  int tau;         // tokens per tile
  int S;           // tokens in the volume (rows of a raster tensor)
  int S_pad;       // n_tiles * tau (rows of a tile-major tensor)
  int padded;      // S_pad != S
};

}  // namespace sta
