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

#include "sta_attn_common.h"

namespace sta {
namespace {

// Per-wave state of the flash loop: Q fragments, O^T accumulators, running
// max m (log2 units) and partial row sums, the current scores and the bf16
// probabilities, and the lane's byte offsets into a K/V buffer.
template <class C, int RB>
struct WaveState {
  typename C::QFrag qf[RB][C::kDK];
  f32x4 o[RB][C::kDB];
  float m[RB], lsum[RB];
  f32x4 s[RB][C::kKT];
  bf16x8 pf[RB][C::kKP];
  // K operand: row 16*kt + l16, chunk 4*dk + g (fp8: chunks 8*dk + 2g and
  // 8*dk + 2g + 1, in koff[2dk] and koff[2dk + 1]); the swizzled offset is
  // koff[.] + 16*kt*row_bytes because the row's low 4 bits are l16.
  int koff[C::kKOffs];
  // V operand (transposing read): row 32*kp + 4g + l16/4 (+16 for the upper
  // half), element column 16*db + 4*(l16 % 4); offset voff[db] + rows*row_bytes.
  int voff[C::kDB];
};

template <class C, int RB>
__device__ __forceinline__ void lane_offsets(WaveState<C, RB>& w, int l16, int g) {
  if constexpr (C::kQK8) {
#pragma unroll
    for (int i = 0; i < C::kKOffs; ++i)
      w.koff[i] = swz<C::KGeom::kCPR>(l16, 8 * (i / 2) + 2 * g + (i % 2));
  } else {
#pragma unroll
    for (int dk = 0; dk < C::kDK; ++dk) w.koff[dk] = swz<C::kCPR>(l16, 4 * dk + g);
  }
  const int s4 = l16 >> 2, sq = l16 & 3;
  const int vrow = 4 * g + s4;  // row within its 16-row group (< 16)
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
    const int col = 16 * db + 4 * sq;
    w.voff[db] = swz<C::kCPR>(vrow, col >> 3) + (col & 7) * 2;
  }
}

// One k-step dk of score tile kt for every row block: sc[.][kt] += K Q^T.
// fp8: a lane's 32 bytes of K are chunks 2g and 2g + 1 of the step's 128
// dimensions, the same dimensions (in the same byte order) as its 32 bytes
// of Q, so the MFMA pairs them whatever order it sums the products in. The
// zero format and scale operands select e4m3 for both and no scaling.
template <class C, int RB>
__device__ __forceinline__ void qk_step(WaveState<C, RB>& w, f32x4 (&sc)[RB][C::kKT], int kt,
                                        int dk, const char* kbuf) {
  if constexpr (C::kQK8) {
    const char* rows = kbuf + 16 * kt * C::KGeom::kRowBytes;
    const i32x4 lo = *reinterpret_cast<const i32x4*>(rows + w.koff[2 * dk]);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(rows + w.koff[2 * dk + 1]);
    const i32x8 kf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      sc[rb][kt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, w.qf[rb][dk], sc[rb][kt],
                                                                    0, 0, 0, 0, 0, 0);
  } else {
    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kbuf + w.koff[dk] + 16 * kt * C::kRowBytes);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      sc[rb][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, w.qf[rb][dk], sc[rb][kt], 0, 0, 0);
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
    for (int dk = 0; dk < C::kDK; ++dk) qk_step<C, RB>(w, sc, kt, dk, kbuf);
  }
}

template <class C, int RB>
__device__ __forceinline__ void qk_chunk(WaveState<C, RB>& w, const char* kbuf, int l16, int g) {
  qk_into<C, RB>(w, w.s, kbuf, l16, g);
}

// Moves each row's reference max to the larger of it and the row's maximum
// (mx: this lane's maximum in log2 units; the row's four lanes are combined
// here) and rescales O and the row sum to match.
template <class C, int RB>
__device__ __forceinline__ void rescale_to(WaveState<C, RB>& w, const float (&mx)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float m_new = fmaxf(w.m[rb], row_max4(mx[rb]));
    const float alpha = __builtin_amdgcn_exp2f(w.m[rb] - m_new);
    w.m[rb] = m_new;
    w.lsum[rb] *= alpha;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) w.o[rb][db] *= alpha;
  }
}

template <class C, int RB>
__device__ __forceinline__ void softmax_max(WaveState<C, RB>& w, f32x4 (&sc)[RB][C::kKT],
                                            int nvalid, unsigned long long real, float scale_log2,
                                            int g) {
  if (nvalid < C::kBN || real != ~0ull) {
    keep_branch();
#pragma unroll
    for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * kt + 4 * g + r;
        if (key >= nvalid || !((real >> key) & 1ull))
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) sc[rb][kt][r] = -INFINITY;
      }
  }
  // The test needs no cross-lane reduction: a row's max exceeds m + 8 exactly
  // when the max of one of its four lanes does, and the decision is taken for
  // the whole wave anyway. Only when it fires is each row's max gathered.
  float mx[RB];
  bool grow = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float a = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::kKT; ++kt)
      a = fmaxf(a, fmaxf(fmaxf(sc[rb][kt][0], sc[rb][kt][1]), fmaxf(sc[rb][kt][2], sc[rb][kt][3])));
    mx[rb] = a * scale_log2;
    grow |= mx[rb] > w.m[rb] + 8.0f;
  }
  if (__any(grow)) {
    keep_branch();
    rescale_to<C, RB>(w, mx);
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
__device__ __forceinline__ void softmax_chunk(WaveState<C, RB>& w, int nvalid,
                                              unsigned long long real, float scale_log2, int g) {
  softmax_max<C, RB>(w, w.s, nvalid, real, scale_log2, g);
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

// Operand reads of an MFMA phase issued AHEAD fragment steps before the
// MFMAs that use them (STEPS steps of DS reads each and RB MFMAs), so that the
// LDS latency runs under earlier MFMAs instead of stalling both waves of a
// SIMD at every fragment (measured: two steps ahead 4-5 % faster than reading
// each fragment just before its MFMAs; three no better).
constexpr int kReadAhead = 2;
template <int RB, int STEPS, int DS, int AHEAD>
__device__ __forceinline__ void sched_reads_ahead() {
#pragma unroll
  for (int st = 0; st < AHEAD && st < STEPS; ++st) __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    if (st + AHEAD < STEPS) __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
  }
}

// ---------------------------------------------------------------------------
// Chunks with every key real: the softmax during QK^T
// ---------------------------------------------------------------------------
// A wave overlaps VALU work only with its own MFMAs, so the probabilities of
// score tile kt (and their row sums) are issued between the QK^T MFMAs of
// tile kt + 1, against the reference max m as it stands. No chunk maximum is
// taken: every probability is at most its lane's sum over the chunk, so a
// lane sum within 2^8 keeps every probability within 2^8, the same bound the
// lazy rescale keeps. A larger (or infinite) sum sends the chunk down a rare
// branch that computes its scores again from LDS, moves m to the exact row
// maximum, rescales O and the row sums, and redoes the probabilities. The
// first chunk of a work item (m = -inf, which would always take that branch)
// runs the max-first order of the masked path instead.

// S^T of score tile kt (keys 16*kt ..) for every row block.
template <class C, int RB>
__device__ __forceinline__ void qk_tile(WaveState<C, RB>& w, int kt, const char* kbuf) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) w.s[rb][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dk = 0; dk < C::kDK; ++dk) qk_step<C, RB>(w, w.s, kt, dk, kbuf);
}

// Probabilities of score tile kt against the reference max, rounded to bf16
// into their slots of the PV operand (tile kt is half kt % 2 of key step kt / 2).
// Log-sum-exp only: the probabilities are summed in fp32 and never rounded.
template <class C, int RB>
__device__ __forceinline__ void exp_sum_tile(WaveState<C, RB>& w, int kt, float scale_log2,
                                             float (&lc)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(w.s[rb][kt][r], scale_log2, -w.m[rb]));
    lc[rb] += (e[0] + e[1]) + (e[2] + e[3]);
  }
}

template <class C, int RB>
__device__ __forceinline__ void exp_tile(WaveState<C, RB>& w, int kt, float scale_log2) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(w.s[rb][kt][r], scale_log2, -w.m[rb]));
#pragma unroll
    for (int r = 0; r < 4; ++r) w.pf[rb][kt / 2][4 * (kt % 2) + r] = static_cast<bf16_t>(e[r]);
  }
}

// Lane sums of the chunk's bf16 probabilities (the values that multiply V).
template <class C, int RB>
__device__ __forceinline__ void chunk_sums(const WaveState<C, RB>& w, float (&lc)[RB]) {
  const bf16x2 ones = {static_cast<bf16_t>(1.0f), static_cast<bf16_t>(1.0f)};
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float ls = 0.f;
#pragma unroll
    for (int kp = 0; kp < C::kKP; ++kp)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {w.pf[rb][kp][2 * e], w.pf[rb][kp][2 * e + 1]};
        ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls, false);
      }
    lc[rb] = ls;
  }
}

// Issue order of the QK^T phase: operand reads three steps ahead; from tile
// 1 on, VPM VALU instructions (of the previous tile's probabilities and
// sums) after each MFMA, the rest where the scheduler puts them. Measured on
// the headline shape against the plain order: with reads two steps ahead,
// two per MFMA 2-2.5 % faster, three or four slower; reads three steps ahead
// another 1.7 % (four: less). Then the kernel that addresses plane chunks
// by arithmetic is 1.3 % faster with one per MFMA than with two (none: 2 %
// slower), while the tile-major kernel is 2 % slower with one than with two.
// RPS: LDS reads per fragment step (2 for fp8 K).
constexpr int kQkReadAhead = 3;
template <int RB, int KT, int DK, int VPM, int RPS = 1>
__device__ __forceinline__ void sched_qk_softmax() {
  constexpr int steps = KT * DK;
#pragma unroll
  for (int st = 0; st < kQkReadAhead && st < steps; ++st) __builtin_amdgcn_sched_group_barrier(0x100, RPS, 0);
#pragma unroll
  for (int st = 0; st < steps; ++st) {
    if (st + kQkReadAhead < steps) __builtin_amdgcn_sched_group_barrier(0x100, RPS, 0);
#pragma unroll
    for (int m = 0; m < RB; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (st >= DK) __builtin_amdgcn_sched_group_barrier(0x402, VPM, 0);   // VALU and transcendental
    }
  }
}

template <bool B>
struct FirstChunk {
  static constexpr bool value = B;
};

// Q rows into registers: bf16, dimensions 32*dk + 8g .. +8 of the lane's row;
// fp8, dimensions 128*dk + 32g .. +32 (the bytes the K reads pair them with).
template <class C, int RB>
__device__ __forceinline__ void load_q_init(WaveState<C, RB>& w, const void* qg,
                                            const RowMap<C, RB>& rm, int l16, int g) {
  lane_offsets<C, RB>(w, l16, g);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if constexpr (C::kQK8) {
      const char* src = static_cast<const char*>(qg) + (long long)rm.tok[rb] * C::kD + 32 * g;
#pragma unroll
      for (int dk = 0; dk < C::kDK; ++dk) {
        i32x8 x = *reinterpret_cast<const i32x8*>(src + 128 * dk);
        if (!rm.ok[rb]) x = i32x8{};
        w.qf[rb][dk] = x;
      }
    } else {
      const bf16_t* src = static_cast<const bf16_t*>(qg) + (long long)rm.tok[rb] * C::kD + 8 * g;
#pragma unroll
      for (int dk = 0; dk < C::kDK; ++dk) {
        bf16x8 x = *reinterpret_cast<const bf16x8*>(src + 32 * dk);
        if (!rm.ok[rb]) x = bf16x8{};
        w.qf[rb][dk] = x;
      }
    }
    w.m[rb] = -INFINITY;
    w.lsum[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) w.o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Normalise and store: lane holds O[row l16][16*db + 4g + r].
template <class C, int RB>
__device__ __forceinline__ void store_out(WaveState<C, RB>& w, bf16_t* og, float* lse,
                                          const RowMap<C, RB>& rm, int g) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l = row_sum4(w.lsum[rb]);
    const float inv = 1.0f / l;
    // log sum_j exp(scale q.k_j) = ln 2 * (m + log2 l), m and l in base 2.
    if (lse && rm.ok[rb] && g == 0) lse[rm.tok[rb]] = (w.m[rb] + __log2f(l)) * kLn2;
    if (og && rm.ok[rb]) {
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

// Flash loop: every wave runs QK^T, softmax and PV of a chunk in turn; the
// next chunk's K and V stream into the other LDS buffer meanwhile (issued
// after QK^T). In both MFMA phases the operand reads run two fragment steps
// ahead of their MFMAs.
// RASTER: q, k, v, out are in raster token order (the permutation to and from
// tile-major order is folded into the addressing): query rows map through
// tile_row_raster, and every key of a window run through a table of raster
// offsets built in dynamic LDS at the start (all runs of a work item share
// it). PLANE (raster, unpadded, tiles whose c_h * c_w plane holds whole
// 64-key chunks): each chunk is BN / c_w rows of c_w consecutive raster
// tokens, addressed by arithmetic, and no table is needed.
// LSE_ONLY: only the row log-sum-exp is wanted (window scoring); V is neither
// loaded nor multiplied and no output is written.
// FULL: every chunk of every work item has BN real keys (no ragged run end,
// no padding): only the spread-out softmax is compiled in; otherwise only the
// masked path (two paths in one kernel would not fit the register file).
// QK8: q and k are fp8 e4m3 (their scales folded into p.scale_log2).
template <int D, int WAVES, int RB, int BN, bool DENSE, bool RASTER, bool LSE_ONLY = false,
          bool PAD = false, bool PLANE = false, bool FULL = false, bool QK8 = false>
__global__ void __launch_bounds__(WAVES * 64, (WAVES <= 4 ? 2 : 1))
attn_bf16_kernel(const AttnParams p) {
  using C = Bf16Cfg<D, WAVES, RB, BN, QK8>;
  using KG = typename C::KGeom;
  // K and V buffers of two chunks. They are separate objects and the loop
  // selects them statically, so the compiler can tell the chunk being read
  // apart from the one the LDS DMA is filling and does not wait for the
  // prefetch before reading.
  __shared__ __attribute__((aligned(1024))) char kb0[KG::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char vb0[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char kb1[KG::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char vb1[C::kChunkBytes];
  // Raster offsets of one window run (RASTER only), sized at launch.
  extern __shared__ int rtab[];

  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<C::kRows>(p, task, D);
  constexpr int kQkBytes = QK8 ? 1 : 2;   // bytes per element of q and k
  const char* qg = static_cast<const char*>(p.q) + t.head_base * kQkBytes;
  const char* kg = static_cast<const char*>(p.k) + t.head_base * kQkBytes;
  const bf16_t* vg = static_cast<const bf16_t*>(p.v) + t.head_base;
  bf16_t* og = static_cast<bf16_t*>(p.out) + t.head_base;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const ChunkWalk walk = make_walk<BN, DENSE>(t, p.S);
  // Plane chunks: raster rows by arithmetic (no table); else the table.
  constexpr bool plane = RASTER && PLANE && BN == 64;
  int lane_row[(C::kBlocks + WAVES - 1) / WAVES];
  int lane_row_k[(KG::kBlocks + WAVES - 1) / WAVES];   // fp8 K rows (QK8 only)
  if constexpr (plane) {
    plane_lane_rows<C, WAVES>(p, wave, lane, lane_row);
    if constexpr (QK8) plane_lane_rows<KG, WAVES>(p, wave, lane, lane_row_k);
  } else if (RASTER) {
    for (int e = threadIdx.x; e < walk.run_len; e += C::kThreads) rtab[e] = run_offset_raster(p, e);
    __syncthreads();
  }
  auto dma = [&](int it, char* kdst, char* vdst) __attribute__((always_inline)) {
    if constexpr (plane) {
      const int row0 = walk.at_plane(p, it);
      if constexpr (QK8)
        load_rows_plane<KG, WAVES>(kg, row0, lane_row_k, kdst, wave, lane);
      else
        load_rows_plane<C, WAVES>(kg, row0, lane_row, kdst, wave, lane);
      if (!LSE_ONLY) load_rows_plane<C, WAVES>(vg, row0, lane_row, vdst, wave, lane);
    } else if (RASTER) {
      int base, c0, nv;
      walk.at_raster(p, it, &base, &c0, &nv);
      const unsigned long long real = chunk_real_keys<PAD>(p, walk, it, lane);
      load_rows<KG, WAVES>(kg, base, nv, kdst, wave, lane, rtab + c0, real);
      if (!LSE_ONLY) load_rows<C, WAVES>(vg, base, nv, vdst, wave, lane, rtab + c0, real);
    } else {
      int row0, nv;
      walk.at(it, &row0, &nv);
      load_rows<KG, WAVES>(kg, row0, nv, kdst, wave, lane);
      if (!LSE_ONLY) load_rows<C, WAVES>(vg, row0, nv, vdst, wave, lane);
    }
  };
  dma(0, kb0, vb0);
  WaveState<C, RB> w;
  load_q_init<C, RB>(w, qg, map_rows<C, RB, RASTER>(p, t, wave, l16), l16, g);

  auto chunk_step = [&](auto first, const char* kcur, const char* vcur, char* knxt, char* vnxt, int it)
                        __attribute__((always_inline)) {
    int row0, nvalid;
    walk.at(it, &row0, &nvalid);
    const unsigned long long real = chunk_real_keys<PAD && !DENSE>(p, walk, it, lane);
    wait_vm_all();     // this wave's loads of chunk `it` have landed in LDS
    __syncthreads();   // ... and every wave's; chunk it-1's buffers are free
    if constexpr (FULL && !decltype(first)::value) {
      float lc[RB];
      if constexpr (LSE_ONLY) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) lc[rb] = 0.f;
#pragma unroll
        for (int kt = 0; kt < C::kKT; ++kt) {
          qk_tile<C, RB>(w, kt, kcur);
          if (kt > 0) exp_sum_tile<C, RB>(w, kt - 1, p.scale_log2, lc);
        }
        exp_sum_tile<C, RB>(w, C::kKT - 1, p.scale_log2, lc);
      } else {
#pragma unroll
        for (int kt = 0; kt < C::kKT; ++kt) {
          qk_tile<C, RB>(w, kt, kcur);
          if (kt > 0) exp_tile<C, RB>(w, kt - 1, p.scale_log2);
        }
        exp_tile<C, RB>(w, C::kKT - 1, p.scale_log2);
        chunk_sums<C, RB>(w, lc);
      }
      // Keep the probabilities and sums here, beside the MFMAs: the compiler
      // would otherwise move them past the branch of the loads below.
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if constexpr (!LSE_ONLY) {
#pragma unroll
          for (int kp = 0; kp < C::kKP; ++kp) asm volatile("" : "+v"(w.pf[rb][kp]));
        }
        asm volatile("" : "+v"(lc[rb]));
      }
      // fp8: one MFMA per tile and row block, twice as long as a bf16 one.
      sched_qk_softmax<RB, C::kKT, C::kDK, (plane ? 1 : 2) * (QK8 ? 2 : 1), QK8 ? 2 : 1>();
      __builtin_amdgcn_sched_barrier(0);
      if (it + 1 < walk.n_chunks) dma(it + 1, knxt, vnxt);
      bool grow = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) grow |= !(lc[rb] <= 256.0f);   // also an infinite sum
      if (__any(grow)) {
        keep_branch();
        qk_chunk<C, RB>(w, kcur, l16, g);
        float mx[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float a = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < C::kKT; ++kt)
            a = fmaxf(a, fmaxf(fmaxf(w.s[rb][kt][0], w.s[rb][kt][1]), fmaxf(w.s[rb][kt][2], w.s[rb][kt][3])));
          mx[rb] = a * p.scale_log2;
        }
        rescale_to<C, RB>(w, mx);
        if constexpr (LSE_ONLY) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) lc[rb] = 0.f;
#pragma unroll
          for (int kt = 0; kt < C::kKT; ++kt) exp_sum_tile<C, RB>(w, kt, p.scale_log2, lc);
        } else {
#pragma unroll
          for (int kt = 0; kt < C::kKT; ++kt) exp_tile<C, RB>(w, kt, p.scale_log2);
          chunk_sums<C, RB>(w, lc);
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) w.lsum[rb] += lc[rb];
      if constexpr (!LSE_ONLY) {
        pv_chunk<C, RB>(w, vcur, l16, g);
        sched_reads_ahead<RB, C::kKP * C::kDB, 2, kReadAhead>();
      }
    } else {
      // Chunks that may hold masked keys (a ragged run end, padding positions).
      qk_chunk<C, RB>(w, kcur, l16, g);
      sched_reads_ahead<RB, C::kKT * C::kDK, QK8 ? 2 : 1, kReadAhead>();
      __builtin_amdgcn_sched_barrier(0);
      // The next chunk's loads go out after QK^T, so their LDS writes land
      // during the softmax (few LDS reads) rather than beside the K reads
      // (measured: 2 % faster than issuing right after the barrier).
      if (it + 1 < walk.n_chunks) dma(it + 1, knxt, vnxt);
      softmax_chunk<C, RB>(w, nvalid, real, p.scale_log2, g);
      // No fence before PV: the scheduler starts the PV MFMAs of the first
      // row block while the exponentials of the others are still being
      // issued (the same wave issuing both is what lets them run side by side).
      if constexpr (!LSE_ONLY) {
        pv_chunk<C, RB>(w, vcur, l16, g);
        sched_reads_ahead<RB, C::kKP * C::kDB, 2, kReadAhead>();
      }
    }
  };
  if constexpr (FULL) {
    // The first chunk sets the reference max: the max-first order, which the
    // sum test would otherwise send down its rare branch every time.
    chunk_step(FirstChunk<true>{}, kb0, vb0, kb1, vb1, 0);
    for (int it = 1; it < walk.n_chunks; it += 2) {
      chunk_step(FirstChunk<false>{}, kb1, vb1, kb0, vb0, it);
      if (it + 1 < walk.n_chunks) chunk_step(FirstChunk<false>{}, kb0, vb0, kb1, vb1, it + 1);
    }
  } else {
    for (int it = 0; it < walk.n_chunks; it += 2) {
      chunk_step(FirstChunk<false>{}, kb0, vb0, kb1, vb1, it);
      if (it + 1 < walk.n_chunks) chunk_step(FirstChunk<false>{}, kb1, vb1, kb0, vb0, it + 1);
    }
  }
  // The row map is built again rather than kept in registers across the loop.
  store_out<C, RB>(w, LSE_ONLY ? nullptr : og, p.lse ? p.lse + t.head_base / D : nullptr,
                   map_rows<C, RB, RASTER>(p, t, wave, l16), g);
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
  float* og = p.out ? static_cast<float*>(p.out) + t.head_base : nullptr;

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
    if (p.lse) p.lse[t.head_base / D + q_tok] = (m + __log2f(l)) * kLn2;
    if (og) {
      float* dst = og + (long long)q_tok * D;
#pragma unroll
      for (int d = 0; d < D; ++d) dst[d] = o[d] * inv;
    }
  }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

void fill_params(const AttnProblem& pr, int rows_per_item, AttnParams* p) {
  p->q = pr.q; p->k = pr.k; p->v = pr.v; p->out = pr.out;
  p->lse = pr.lse;
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
  } else {
    p->n_units = pr.g.n_tiles;
    p->unit_rows = pr.g.tau;
    p->nt = pr.g.nt; p->nh = pr.g.nh; p->nw = pr.g.nw;
    p->tau = pr.g.tau;
    p->T = pr.g.T; p->H = pr.g.H; p->W = pr.g.W;
    p->ct = pr.g.ct; p->ch = pr.g.ch; p->cw = pr.g.cw;
    p->pad = pr.g.padded;
    set_plane_chunks(p);
    for (int h = 0; h < pr.heads; ++h)
      for (int a = 0; a < 3; ++a) p->omega[h][a] = pr.omega[h][a];
  }
  p->row_blocks = (p->unit_rows + rows_per_item - 1) / rows_per_item;
  const long long tasks = (long long)pr.B * pr.heads * p->n_units * p->row_blocks;
  plan_tasks(p, tasks, pr.heads, pr.dense);
}

// LDS for the raster offsets of the longest window run, omega_w * tau keys.
unsigned raster_table_bytes(const AttnProblem& pr) {
  int run = 0;
  for (int h = 0; h < pr.heads; ++h) run = pr.omega[h][2] * pr.g.tau > run ? pr.omega[h][2] * pr.g.tau : run;
  return (unsigned)run * sizeof(int);
}

// FULL implies !PAD; plane chunks imply FULL (whole 64-key chunks per tile).
// QK8 (fp8 q and k) has no log-sum-exp-only form; the host never asks for one.
template <int D, int WAVES, int RB, int BN, bool PAD, bool FULL, bool QK8>
void launch_sparse(const AttnProblem& pr, const AttnParams& p, unsigned grid, unsigned table,
                   hipStream_t stream) {
  using C = Bf16Cfg<D, WAVES, RB, BN>;
  const bool plane = FULL && BN == 64 && p.plane_cpt > 0;
  if constexpr (QK8) {
    if (pr.raster && plane)
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, true, false, false, true, true, true>),
                         dim3(grid), dim3(C::kThreads), 0, stream, p);
    else if (pr.raster)
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, true, false, PAD, false, FULL, true>),
                         dim3(grid), dim3(C::kThreads), table, stream, p);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, false, false, PAD, false, FULL, true>),
                         dim3(grid), dim3(C::kThreads), 0, stream, p);
  } else if (pr.lse_only) {
    if constexpr (FULL) {
      if (pr.raster && plane) {
        hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, true, true, false, true, true>),
                           dim3(grid), dim3(C::kThreads), 0, stream, p);
        return;
      }
    }
    if (pr.raster)
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, true, true, PAD, false, FULL>),
                         dim3(grid), dim3(C::kThreads), table, stream, p);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, false, true, PAD, false, FULL>),
                         dim3(grid), dim3(C::kThreads), 0, stream, p);
  } else {
    if constexpr (FULL) {
      if (pr.raster && plane) {
        hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, true, false, false, true, true>),
                           dim3(grid), dim3(C::kThreads), 0, stream, p);
        return;
      }
    }
    if (pr.raster)
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, true, false, PAD, false, FULL>),
                         dim3(grid), dim3(C::kThreads), table, stream, p);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false, false, false, PAD, false, FULL>),
                         dim3(grid), dim3(C::kThreads), 0, stream, p);
  }
}

// Whether every chunk of every work item holds BN keys that are all tokens.
bool chunks_full(const AttnProblem& pr, int bn) {
  if (pr.dense) return pr.g.S % bn == 0;
  if (pr.g.padded) return false;
  for (int h = 0; h < pr.heads; ++h)
    if ((pr.omega[h][2] * pr.g.tau) % bn != 0) return false;
  return true;
}

template <int D, int WAVES, int RB, int BN, bool QK8>
int launch_bf16(const AttnProblem& pr, hipStream_t stream) {
  using C = Bf16Cfg<D, WAVES, RB, BN>;
  AttnParams p;
  fill_params(pr, C::kRows, &p);
  const unsigned grid = (unsigned)p.per_xcd * kXcds;
  // plane chunks address K/V by arithmetic and need no offset table
  const bool full = chunks_full(pr, BN);
  const unsigned table = (full && BN == 64 && p.plane_cpt > 0) ? 0 : raster_table_bytes(pr);
  if constexpr (QK8) {
    if (pr.dense || pr.lse_only) return STA_ERR_UNSUPPORTED;
    if (pr.g.padded)
      launch_sparse<D, WAVES, RB, BN, true, false, true>(pr, p, grid, table, stream);
    else if (full)
      launch_sparse<D, WAVES, RB, BN, false, true, true>(pr, p, grid, table, stream);
    else
      launch_sparse<D, WAVES, RB, BN, false, false, true>(pr, p, grid, table, stream);
    return (int)hipGetLastError();
  }
  if (pr.dense) {
    if (pr.lse_only && full)
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, true, false, true, false, false, true>),
                         dim3(grid), dim3(C::kThreads), 0, stream, p);
    else if (pr.lse_only)
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, true, false, true>), dim3(grid),
                         dim3(C::kThreads), 0, stream, p);
    else if (full)
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, true, false, false, false, false, true>),
                         dim3(grid), dim3(C::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, true, false>), dim3(grid),
                         dim3(C::kThreads), 0, stream, p);
  } else if (pr.g.padded) {
    launch_sparse<D, WAVES, RB, BN, true, false, false>(pr, p, grid, table, stream);
  } else if (full) {
    launch_sparse<D, WAVES, RB, BN, false, true, false>(pr, p, grid, table, stream);
  } else {
    launch_sparse<D, WAVES, RB, BN, false, false, false>(pr, p, grid, table, stream);
  }
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
template <int D, bool QK8 = false>
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
  if (unit_rows % kBigRows == 0)
    return launch_bf16<D, STA_CFG_WAVES, STA_CFG_RB, STA_CFG_BN, QK8>(pr, stream);
  if (unit_rows <= 64) return launch_bf16<D, 4, 1, 64, QK8>(pr, stream);
  return launch_bf16<D, 4, 2, 64, QK8>(pr, stream);
}

}  // namespace

int launch_attention(const AttnProblem& pr, void* stream_ptr) {
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const long long units = pr.dense ? 1 : pr.g.n_tiles;
  const long long tasks_upper = (long long)pr.B * pr.heads * units * (pr.dense ? pr.g.S : pr.g.tau);
  if (tasks_upper > (1LL << 31) - 1) return (int)hipErrorInvalidValue;
  if (pr.qk_fp8) {
    if (pr.dtype == STA_BF16 && pr.head_dim == 128) return dispatch_bf16<128, true>(pr, stream);
    return STA_ERR_UNSUPPORTED;
  }
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
