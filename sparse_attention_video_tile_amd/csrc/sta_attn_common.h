// Device-side building blocks shared by the attention kernels of libsta
// (forward in sta_attention.hip, backward in sta_backward.hip): cross-lane
// reductions, the LDS layout of K/V-like chunks and their direct-to-LDS
// loads, row maps and key masks. The work plan (kernel parameters, work-item
// decoding, the window walk, raster-order addressing) is in sta_plan.h.
//
// Included only by HIP translation units; everything sits in an anonymous
// namespace, so each includer gets its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "sta_kernels.h"
#include "sta_plan.h"

namespace sta {
namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// The logical task of this workgroup (task_of_block).
__device__ __forceinline__ int logical_task(const AttnParams& p) { return task_of_block(p, blockIdx.x); }

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

// This lane's streamed rows of a chunk that are tokens: bit 4*kt + r for row
// 16*kt + 4g + r of the chunk (the rows a lane holds in a 16x16 MFMA result
// tile kt, lane = l16 + 16g), from the chunk's token mask `real` and its row
// count nvalid.
__device__ __forceinline__ unsigned lane_key_mask(unsigned long long real, int nvalid, int g) {
  const unsigned long long v = nvalid >= 64 ? real : real & ((1ull << nvalid) - 1ull);
  const unsigned long long x = v >> (4 * g);
  unsigned km = 0;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) km |= (unsigned)((x >> (16 * kt)) & 0xFull) << (4 * kt);
  return km;
}

// Initial accumulator of score tile kt: 0 for this lane's rows that are
// tokens, -inf for the others. The MFMAs add finite products (such rows load a
// token's row), so their scores come out -inf and their probabilities 0,
// with no test after the products.
__device__ __forceinline__ f32x4 key_bias(unsigned km, int kt) {
  f32x4 b;
#pragma unroll
  for (int r = 0; r < 4; ++r) b[r] = ((km >> (4 * kt + r)) & 1u) ? 0.f : -INFINITY;
  return b;
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


// Bit k set iff key k (0..63) of chunk `it` is a token of the volume: all
// ones unless the problem is padded (PAD, a kernel variant of its own so that
// unpadded launches carry no masking code) and the chunk's run reaches past
// the volume. From the precomputed masks when tau is a multiple of 64, else
// one key per lane (64-key chunks), then a wave ballot.
template <bool PAD>
__device__ __forceinline__ unsigned long long chunk_real_keys(const AttnParams& p, const ChunkWalk& w,
                                                               int it, int lane) {
  if (!PAD) return ~0ull;
  if (p.pad_cpt > 0 && w.bn == 64) return chunk_pad_mask(p, w.kv, w.chunks_per_run, it);
  const int run = it / w.chunks_per_run;
  if (!run_padded(p, w.kv, run)) return ~0ull;
  const int e = (it - run * w.chunks_per_run) * w.bn + lane;
  const bool real = e < w.run_len && run_key_real(p, w.kv, run, e);
  return __ballot(real);
}


}  // namespace
}  // namespace sta
