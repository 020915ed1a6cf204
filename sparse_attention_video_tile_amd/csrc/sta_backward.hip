// Backward kernels of libsta (gfx950): gradients of Sliding Tile Attention.
//
// With P the row softmax of scale * Q K^T over each query's window keys and
// O = P V, the gradients are
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = dO_i . O_i,
//     dQ = scale * dS K,  dK = scale * dS^T Q,
// and P is recomputed from the forward's log-sum-exp: P_ij = exp(scale *
// q_i . k_j - lse_i). Three launches on the caller's stream:
//   1. delta_kernel: D per query row from dO and O.
//   2. dkdv kernel: one work item per block of key rows of one key tile; it
//      walks the query tiles whose window holds that key tile (the window
//      relation transposed; per axis an interval, see window_inverse) and
//      accumulates dK and dV in registers. No atomics.
//   3. dq kernel: one work item per block of query rows of one query tile; it
//      walks the tile's window like the forward and accumulates dQ.
// Each dQ, dK, dV element is written by exactly one work item, so results are
// deterministic.
//
// bf16 kernels use v_mfma_f32_16x16x32_bf16 with the forward's conventions:
// a wave keeps its own rows (queries for dq, keys for dkdv) in registers as
// the B operand, the streamed side sits in LDS in the swizzled chunk layout
// and is read either row-wise (A operand, one 16-byte read per lane) or
// transposed (ds_read_b64_tr_b16); every lane then holds values of one own
// row, and the recomputed P and dS are rounded to bf16 as MFMA operands.
//
// f32 kernels (float32 problems): 32 own rows an item, two lanes a row, the
// walk's 32-row chunks dealt to the waves of the workgroup, whose partial
// gradients add up through LDS at the end.
#include <hip/hip_runtime.h>

#include "sta_attn_common.h"

namespace sta {
namespace {


// ---------------------------------------------------------------------------
// D = rowsum(dO * O)
// ---------------------------------------------------------------------------

// One lane per 16-byte chunk of a row; the CPR lanes of a row reduce with
// butterfly shuffles. rows = B * heads * S (order-agnostic).
template <typename T, int D>
__global__ void __launch_bounds__(256) delta_kernel(const T* o, const T* dout, float* delta,
                                                    long long rows) {
  constexpr int kPer = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int kCPR = D / kPer;         // chunks per row (8..32, a power of two)
  const long long chunk = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = chunk / kCPR;
  float acc = 0.f;
  if (row < rows) {
    const T* a = o + chunk * kPer;
    const T* b = dout + chunk * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc = fmaf(static_cast<float>(a[e]), static_cast<float>(b[e]), acc);
  }
#pragma unroll
  for (int m = kCPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && (threadIdx.x % kCPR) == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// bf16 building blocks
// ---------------------------------------------------------------------------

// Lane offsets into a swizzled chunk buffer: koff for the row-wise operand
// read (row 16*kt + l16, 16-byte piece 4*dk + g), voff for the transposing
// read (row 32*kp + 4g + l16/4 (+16), columns 16*db + 4*(l16 % 4) .. +4).
template <class C>
__device__ __forceinline__ void lane_koff(int (&koff)[C::kDK], int l16, int g) {
#pragma unroll
  for (int dk = 0; dk < C::kDK; ++dk) koff[dk] = swz<C::kCPR>(l16, 4 * dk + g);
}

template <class C>
__device__ __forceinline__ void lane_voff(int (&voff)[C::kDB], int l16, int g) {
  const int s4 = l16 >> 2, sq = l16 & 3;
  const int vrow = 4 * g + s4;
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
    const int col = 16 * db + 4 * sq;
    voff[db] = swz<C::kCPR>(vrow, col >> 3) + (col & 7) * 2;
  }
}

// acc[rb][kt] = X Y^T for one chunk: X = the buffer's rows (16*kt ..), Y = the
// wave's own rows held as fragments fr. Lane (l16, g) receives buffer rows
// 16*kt + 4g + r against own row l16 of block rb. MASK: buffer rows outside
// the lane's token mask km start at -inf, so their scores are -inf.
template <class C, int RB, bool MASK = false>
__device__ __forceinline__ void mma_rows(f32x4 (&acc)[RB][C::kKT], const char* buf,
                                         const int (&koff)[C::kDK],
                                         const bf16x8 (&fr)[RB][C::kDK], unsigned km = 0) {
#pragma unroll
  for (int kt = 0; kt < C::kKT; ++kt) {
    const f32x4 init = MASK ? key_bias(km, kt) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][kt] = init;
#pragma unroll
    for (int dk = 0; dk < C::kDK; ++dk) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(buf + koff[dk] + 16 * kt * C::kRowBytes);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, fr[rb][dk], acc[rb][kt], 0, 0, 0);
    }
  }
}

// acc[rb][db] += X^T W for one chunk: X = the buffer (read transposed), W =
// bf16 weights per (buffer row, own row) packed by pack_bf16. Lane (l16, g)
// accumulates columns 16*db + 4g + r of own row l16. Slot j of lane group g
// is buffer row 32*kp + 4g + j (j < 4) or 32*kp + 16 + 4g + (j - 4), matching
// the transposing read's lane mapping.
template <class C, int RB>
__device__ __forceinline__ void mma_tr(f32x4 (&acc)[RB][C::kDB], const char* buf,
                                       const int (&voff)[C::kDB], const bf16x8 (&wf)[RB][C::kKP]) {
#pragma unroll
  for (int kp = 0; kp < C::kKP; ++kp) {
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) {
      const char* lo_addr = buf + voff[db] + 32 * kp * C::kRowBytes;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(lo_addr));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(lo_addr + 16 * C::kRowBytes));
      const i16x4 both[2] = {lo, hi};
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(both);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, wf[rb][kp], acc[rb][db], 0, 0, 0);
    }
  }
}

template <class C, int RB>
__device__ __forceinline__ void pack_bf16(bf16x8 (&wf)[RB][C::kKP], const f32x4 (&x)[RB][C::kKT]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int kp = 0; kp < C::kKP; ++kp)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wf[rb][kp][r] = static_cast<bf16_t>(x[rb][2 * kp][r]);
        wf[rb][kp][4 + r] = static_cast<bf16_t>(x[rb][2 * kp + 1][r]);
      }
}

// The wave's own rows as B-operand fragments: row l16 of block rb, 16-byte
// piece 4*dk + g. Rows that do not exist read row 0 of the unit and are
// zeroed.
template <class C, int RB>
__device__ __forceinline__ void load_frags(bf16x8 (&fr)[RB][C::kDK], const bf16_t* src,
                                           const RowMap<C, RB>& rm, int g) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bf16_t* row = src + (long long)rm.tok[rb] * C::kD + 8 * g;
#pragma unroll
    for (int dk = 0; dk < C::kDK; ++dk) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(row + 32 * dk);
      if (!rm.ok[rb]) x = bf16x8{};
      fr[rb][dk] = x;
    }
  }
}

// Stores own-row accumulators (lane: columns 16*db + 4g + r of row l16) times
// `mul` as bf16.
template <class C, int RB>
__device__ __forceinline__ void store_rows(const f32x4 (&acc)[RB][C::kDB], bf16_t* dst_base,
                                           const RowMap<C, RB>& rm, int g, float mul) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!rm.ok[rb]) continue;
    bf16_t* dst = dst_base + (long long)rm.tok[rb] * C::kD + 4 * g;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) {
      bf16x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = static_cast<bf16_t>(acc[rb][db][e] * mul);
      *reinterpret_cast<bf16x4*>(dst + 16 * db) = y;
    }
  }
}

// One float per streamed row of a chunk (lse or D) into LDS with a single
// direct-to-LDS dword load: lane i fills slot i (BN = 64 rows, one wave).
__device__ __forceinline__ void load_row_values(const float* src, int row0, int nvalid, float* buf,
                                                int lane, const int* rtab, unsigned long long real,
                                                int key_base) {
  const int key = min(lane, nvalid - 1);
  int rel = rtab ? rtab[key] : key_base + key;
  if (!((real >> key) & 1ull)) rel = 0;
  lds_dma<4>(src + __builtin_amdgcn_readfirstlane(row0), rel * 4, buf);
}

// Operand reads of an MFMA phase issued AHEAD steps before the MFMAs that use
// them (each step: DS reads, then RB MFMAs); VALU work from an earlier phase
// may fill VPM instructions after each MFMA. Measured at the headline shape:
// three steps ahead for the row-wise reads and two for the transposing ones,
// three VALU instructions per MFMA where there is VALU work to place.
template <int RB, int STEPS, int DS, int AHEAD, int VPM>
__device__ __forceinline__ void sched_phase() {
#pragma unroll
  for (int st = 0; st < AHEAD && st < STEPS; ++st) __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    if (st + AHEAD < STEPS) __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
#pragma unroll
    for (int m = 0; m < RB; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (VPM > 0) __builtin_amdgcn_sched_group_barrier(0x402, VPM, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// dq kernel (own rows: queries; streamed: K and V of the window)
// ---------------------------------------------------------------------------

template <int D, int WAVES, int RB, int BN, bool RASTER, bool PAD, bool FULL>
__global__ void __launch_bounds__(WAVES * 64, (WAVES <= 4 ? 2 : 1))
bwd_dq_kernel(const AttnParams p, const BwdParams b) {
  using C = Bf16Cfg<D, WAVES, RB, BN>;
  __shared__ __attribute__((aligned(1024))) char kb0[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char vb0[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char kb1[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char vb1[C::kChunkBytes];
  extern __shared__ int rtab[];

  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<C::kRows>(p, task, D);
  const long long rowbase = t.head_base / D;
  const bf16_t* qg = static_cast<const bf16_t*>(p.q) + t.head_base;
  const bf16_t* kg = static_cast<const bf16_t*>(p.k) + t.head_base;
  const bf16_t* vg = static_cast<const bf16_t*>(p.v) + t.head_base;
  const bf16_t* dog = static_cast<const bf16_t*>(b.dout) + t.head_base;
  bf16_t* dqg = static_cast<bf16_t*>(b.dq) + t.head_base;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const ChunkWalk walk = make_walk<BN, false>(t, p.S);
  if (RASTER) {
    for (int e = threadIdx.x; e < walk.run_len; e += C::kThreads) rtab[e] = run_offset_raster(p, e);
    __syncthreads();
  }
  auto dma = [&](int it, char* kdst, char* vdst) __attribute__((always_inline)) {
    if (RASTER) {
      int base, c0, nv;
      walk.at_raster(p, it, &base, &c0, &nv);
      const unsigned long long real = chunk_real_keys<PAD>(p, walk, it, lane);
      load_rows<C, WAVES>(kg, base, nv, kdst, wave, lane, rtab + c0, real);
      load_rows<C, WAVES>(vg, base, nv, vdst, wave, lane, rtab + c0, real);
    } else if constexpr (PAD) {
      int row0, kb, nv;
      walk.at_tile(it, p.tau, &row0, &kb, &nv);
      const unsigned long long real = chunk_real_keys<PAD>(p, walk, it, lane);
      load_rows<C, WAVES>(kg, row0, nv, kdst, wave, lane, nullptr, real, kb);
      load_rows<C, WAVES>(vg, row0, nv, vdst, wave, lane, nullptr, real, kb);
    } else {
      int row0, nv;
      walk.at(it, &row0, &nv);
      load_rows<C, WAVES>(kg, row0, nv, kdst, wave, lane);
      load_rows<C, WAVES>(vg, row0, nv, vdst, wave, lane);
    }
  };
  dma(0, kb0, vb0);

  const RowMap<C, RB> rm = map_rows<C, RB, RASTER>(p, t, wave, l16);
  int koff[C::kDK], voff[C::kDB];
  lane_koff<C>(koff, l16, g);
  lane_voff<C>(voff, l16, g);
  bf16x8 qf[RB][C::kDK], df[RB][C::kDK];
  load_frags<C, RB>(qf, qg, rm, g);
  load_frags<C, RB>(df, dog, rm, g);
  float lse2[RB], dl[RB];
  f32x4 acc[RB][C::kDB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lse2[rb] = rm.ok[rb] ? b.lse[rowbase + rm.tok[rb]] * kLog2e : 0.f;
    dl[rb] = rm.ok[rb] ? b.delta[rowbase + rm.tok[rb]] : 0.f;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto chunk_step = [&](const char* kcur, const char* vcur, char* knxt, char* vnxt, int it)
                        __attribute__((always_inline)) {
    int row0, nvalid;
    walk.at(it, &row0, &nvalid);
    wait_vm_all();
    __syncthreads();
    const unsigned long long real = chunk_real_keys<PAD>(p, walk, it, lane);
    // keys that are not tokens (padding, a ragged run end) score -inf: their
    // P^T and dS^T come out 0 (their K and V rows are a token's, finite)
    const unsigned km = FULL ? 0u : lane_key_mask(real, nvalid, g);
    f32x4 s[RB][C::kKT], dp[RB][C::kKT];
    mma_rows<C, RB, !FULL>(s, kcur, koff, qf, km);    // S^T[key][row] = K Q^T
    sched_phase<RB, C::kKT * C::kDK, 1, 3, 0>();
    // P^T while dP^T = V dO^T runs
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s[rb][kt][r] = __builtin_amdgcn_exp2f(fmaf(s[rb][kt][r], p.scale_log2, -lse2[rb]));
    mma_rows<C, RB>(dp, vcur, koff, df);   // dP^T[key][row] = V dO^T
    sched_phase<RB, C::kKT * C::kDK, 1, 3, 3>();
    __builtin_amdgcn_sched_barrier(0);
    // next chunk's loads after the row-wise reads
    if (it + 1 < walk.n_chunks) dma(it + 1, knxt, vnxt);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s[rb][kt][r] = s[rb][kt][r] * (dp[rb][kt][r] - dl[rb]);   // dS^T
    bf16x8 wf[RB][C::kKP];
    pack_bf16<C, RB>(wf, s);
    mma_tr<C, RB>(acc, kcur, voff, wf);    // dQ^T[d][row] += K^T dS^T
    sched_phase<RB, C::kKP * C::kDB, 2, 2, 0>();
  };
  for (int it = 0; it < walk.n_chunks; it += 2) {
    chunk_step(kb0, vb0, kb1, vb1, it);
    if (it + 1 < walk.n_chunks) chunk_step(kb1, vb1, kb0, vb0, it + 1);
  }
  store_rows<C, RB>(acc, dqg, rm, g, b.scale);
}

// ---------------------------------------------------------------------------
// dkdv kernel (own rows: keys; streamed: Q, dO, lse and D of the query tiles
// whose window holds the key tile)
// ---------------------------------------------------------------------------

template <int D, int WAVES, int RB, int BN, bool RASTER, bool PAD, bool FULL>
__global__ void __launch_bounds__(WAVES * 64, (WAVES <= 4 ? 2 : 1))
bwd_dkdv_kernel(const AttnParams p, const BwdParams b) {
  using C = Bf16Cfg<D, WAVES, RB, BN>;
  static_assert(BN == 64, "one wave loads the chunk's lse and D rows");
  __shared__ __attribute__((aligned(1024))) char qb0[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char ob0[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char qb1[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char ob1[C::kChunkBytes];
  __shared__ __attribute__((aligned(256))) float lb0[BN];
  __shared__ __attribute__((aligned(256))) float db0[BN];
  __shared__ __attribute__((aligned(256))) float lb1[BN];
  __shared__ __attribute__((aligned(256))) float db1[BN];
  extern __shared__ int rtab[];

  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<C::kRows, true>(p, task, D);
  const long long rowbase = t.head_base / D;
  const bf16_t* qg = static_cast<const bf16_t*>(p.q) + t.head_base;
  const bf16_t* kg = static_cast<const bf16_t*>(p.k) + t.head_base;
  const bf16_t* vg = static_cast<const bf16_t*>(p.v) + t.head_base;
  const bf16_t* dog = static_cast<const bf16_t*>(b.dout) + t.head_base;
  const float* lseg = b.lse + rowbase;
  const float* delg = b.delta + rowbase;
  bf16_t* dkg = static_cast<bf16_t*>(b.dk) + t.head_base;
  bf16_t* dvg = static_cast<bf16_t*>(b.dv) + t.head_base;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const ChunkWalk walk = make_walk<BN, false>(t, p.S);
  if (RASTER) {
    for (int e = threadIdx.x; e < walk.run_len; e += C::kThreads) rtab[e] = run_offset_raster(p, e);
    __syncthreads();
  }
  auto dma = [&](int it, char* qdst, char* odst, float* ldst, float* ddst)
                 __attribute__((always_inline)) {
    int base, c0 = 0, nv;
    const int* tab = nullptr;
    if (RASTER) {
      walk.at_raster(p, it, &base, &c0, &nv);
      tab = rtab + c0;
    } else if (PAD) {
      walk.at_tile(it, p.tau, &base, &c0, &nv);   // padding rows load the tile's first row
    } else {
      walk.at(it, &base, &nv);
    }
    const int kb = RASTER ? 0 : c0;
    const unsigned long long real = chunk_real_keys<PAD>(p, walk, it, lane);
    load_rows<C, WAVES>(qg, base, nv, qdst, wave, lane, tab, real, kb);
    load_rows<C, WAVES>(dog, base, nv, odst, wave, lane, tab, real, kb);
    if (wave == 0) {
      load_row_values(lseg, base, nv, ldst, lane, tab, real, kb);
      load_row_values(delg, base, nv, ddst, lane, tab, real, kb);
    }
  };
  dma(0, qb0, ob0, lb0, db0);

  const RowMap<C, RB> rm = map_rows<C, RB, RASTER>(p, t, wave, l16);
  int koff[C::kDK], voff[C::kDB];
  lane_koff<C>(koff, l16, g);
  lane_voff<C>(voff, l16, g);
  bf16x8 kf[RB][C::kDK], vf[RB][C::kDK];
  load_frags<C, RB>(kf, kg, rm, g);
  load_frags<C, RB>(vf, vg, rm, g);
  f32x4 dk[RB][C::kDB], dv[RB][C::kDB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) {
      dk[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  auto chunk_step = [&](const char* qcur, const char* ocur, const float* lcur, const float* dcur,
                        char* qnxt, char* onxt, float* lnxt, float* dnxt, int it)
                        __attribute__((always_inline)) {
    int row0, nvalid;
    walk.at(it, &row0, &nvalid);
    wait_vm_all();
    __syncthreads();
    const unsigned long long real = chunk_real_keys<PAD>(p, walk, it, lane);
    // query rows that are not tokens score -inf: their P and dS come out 0
    // (their Q, dO, lse and D are a token's, finite)
    const unsigned km = FULL ? 0u : lane_key_mask(real, nvalid, g);
    f32x4 s[RB][C::kKT];
    mma_rows<C, RB, !FULL>(s, qcur, koff, kf, km);    // S[q][key] = Q K^T
    sched_phase<RB, C::kKT * C::kDK, 1, 3, 0>();
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < walk.n_chunks) dma(it + 1, qnxt, onxt, lnxt, dnxt);
    f32x4 lq[C::kKT], dq_[C::kKT];
#pragma unroll
    for (int kt = 0; kt < C::kKT; ++kt) {
      lq[kt] = *reinterpret_cast<const f32x4*>(lcur + 16 * kt + 4 * g);
      dq_[kt] = *reinterpret_cast<const f32x4*>(dcur + 16 * kt + 4 * g);
    }
    // P while dP = dO V^T runs
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)   // P[q][key]
          s[rb][kt][r] = __builtin_amdgcn_exp2f(fmaf(s[rb][kt][r], p.scale_log2, -lq[kt][r] * kLog2e));
    bf16x8 wf[RB][C::kKP];
    pack_bf16<C, RB>(wf, s);
    f32x4 dp[RB][C::kKT];
    mma_rows<C, RB>(dp, ocur, koff, vf);   // dP[q][key] = dO V^T
    sched_phase<RB, C::kKT * C::kDK, 1, 3, 3>();
    // dS while dV^T += dO^T P runs
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)   // dS
          s[rb][kt][r] = s[rb][kt][r] * (dp[rb][kt][r] - dq_[kt][r]);
    bf16x8 wd[RB][C::kKP];
    pack_bf16<C, RB>(wd, s);
    mma_tr<C, RB>(dv, ocur, voff, wf);     // dV^T[d][key] += dO^T P
    sched_phase<RB, C::kKP * C::kDB, 2, 2, 3>();
    mma_tr<C, RB>(dk, qcur, voff, wd);     // dK^T[d][key] += Q^T dS
    sched_phase<RB, C::kKP * C::kDB, 2, 2, 0>();
  };
  for (int it = 0; it < walk.n_chunks; it += 2) {
    chunk_step(qb0, ob0, lb0, db0, qb1, ob1, lb1, db1, it);
    if (it + 1 < walk.n_chunks) chunk_step(qb1, ob1, lb1, db1, qb0, ob0, lb0, db0, it + 1);
  }
  store_rows<C, RB>(dk, dkg, rm, g, b.scale);
  store_rows<C, RB>(dv, dvg, rm, g, 1.0f);
}

// ---------------------------------------------------------------------------
// dkdv kernel with paired waves (own rows: keys, 16 * RB per pair)
// ---------------------------------------------------------------------------
// The one-wave-per-16-keys kernel above reads every streamed Q and dO
// fragment from LDS for a single MFMA, twice per chunk (row-wise and
// transposed), which makes the LDS, not the matrix cores, its bound. Here a
// pair of waves shares 16 * RB key rows and splits the four products:
//   wave P (waves 0 .. PAIRS-1):  S = Q K^T, P = exp(S - lse),   dV^T += dO^T P
//   wave S (waves PAIRS ..):      dP = dO V^T, dS = P * (dP - D), dK^T += Q^T dS
// Each wave issues the same number of MFMAs as before, but every fragment it
// reads feeds RB of them. Wave S takes P from wave P through LDS (bf16, the
// values wave P multiplies dO by), after a second barrier per chunk; wave S
// reads it before it reaches the next chunk's first barrier, so one P buffer
// per pair suffices.
template <int D, int PAIRS, int RB, int BN, bool RASTER, bool PAD, bool FULL>
__global__ void __launch_bounds__(2 * PAIRS * 64, 1)
bwd_dkdv_pair_kernel(const AttnParams p, const BwdParams b) {
  constexpr int WAVES = 2 * PAIRS;
  using C = Bf16Cfg<D, WAVES, RB, BN>;
  static_assert(BN == 64, "one wave loads the chunk's lse and D rows");
  constexpr int kRows = PAIRS * 16 * RB;   // key rows per work item
  __shared__ __attribute__((aligned(1024))) char qb0[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char ob0[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char qb1[C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char ob1[C::kChunkBytes];
  __shared__ __attribute__((aligned(256))) float lb0[BN];
  __shared__ __attribute__((aligned(256))) float db0[BN];
  __shared__ __attribute__((aligned(256))) float lb1[BN];
  __shared__ __attribute__((aligned(256))) float db1[BN];
  // P of the current chunk per pair: slot j (rb * kKP + kp) of lane l at
  // pbuf[pair][j][l], 16 bytes each (contiguous per instruction).
  __shared__ __attribute__((aligned(1024))) bf16x8 pbuf[PAIRS][RB * C::kKP][64];
  extern __shared__ int rtab[];

  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<kRows, true>(p, task, D);
  const long long rowbase = t.head_base / D;
  const bf16_t* qg = static_cast<const bf16_t*>(p.q) + t.head_base;
  const bf16_t* kg = static_cast<const bf16_t*>(p.k) + t.head_base;
  const bf16_t* vg = static_cast<const bf16_t*>(p.v) + t.head_base;
  const bf16_t* dog = static_cast<const bf16_t*>(b.dout) + t.head_base;
  const float* lseg = b.lse + rowbase;
  const float* delg = b.delta + rowbase;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wave % PAIRS;
  const bool wave_p = wave < PAIRS;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const ChunkWalk walk = make_walk<BN, false>(t, p.S);
  if (RASTER) {
    for (int e = threadIdx.x; e < walk.run_len; e += C::kThreads) rtab[e] = run_offset_raster(p, e);
    __syncthreads();
  }
  auto dma = [&](int it, char* qdst, char* odst, float* ldst, float* ddst)
                 __attribute__((always_inline)) {
    int base, c0 = 0, nv;
    const int* tab = nullptr;
    if (RASTER) {
      walk.at_raster(p, it, &base, &c0, &nv);
      tab = rtab + c0;
    } else if (PAD) {
      walk.at_tile(it, p.tau, &base, &c0, &nv);   // padding rows load the tile's first row
    } else {
      walk.at(it, &base, &nv);
    }
    const int kb = RASTER ? 0 : c0;
    const unsigned long long real = chunk_real_keys<PAD>(p, walk, it, lane);
    load_rows<C, WAVES>(qg, base, nv, qdst, wave, lane, tab, real, kb);
    load_rows<C, WAVES>(dog, base, nv, odst, wave, lane, tab, real, kb);
    if (wave == 0) {
      load_row_values(lseg, base, nv, ldst, lane, tab, real, kb);
      load_row_values(delg, base, nv, ddst, lane, tab, real, kb);
    }
  };
  dma(0, qb0, ob0, lb0, db0);

  // Own key rows: rows 16 * RB * pair + 16 * rb + l16 of the work item.
  const RowMap<C, RB> rm = map_rows<C, RB, RASTER>(p, t, pair, l16);
  int koff[C::kDK], voff[C::kDB];
  lane_koff<C>(koff, l16, g);
  lane_voff<C>(voff, l16, g);

  if (wave_p) {
    bf16x8 kf[RB][C::kDK];
    load_frags<C, RB>(kf, static_cast<const bf16_t*>(kg), rm, g);
    f32x4 dv[RB][C::kDB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) dv[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto step = [&](const char* qcur, const char* ocur, const float* lcur, char* qnxt, char* onxt,
                    float* lnxt, float* dnxt, int it) __attribute__((always_inline)) {
      int row0, nvalid;
      walk.at(it, &row0, &nvalid);
      wait_vm_all();
      __syncthreads();
      // the next chunk's loads go out as soon as its buffers are free
      // (measured: 4 % faster on the whole backward than after the first
      // products, 2.5 % than after the mid-chunk barrier)
      if (it + 1 < walk.n_chunks) dma(it + 1, qnxt, onxt, lnxt, dnxt);
      const unsigned long long real = chunk_real_keys<PAD>(p, walk, it, lane);
      // query rows that are not tokens score -inf, so their P is 0 (and so
      // is wave S's dS, which multiplies P)
      const unsigned km = FULL ? 0u : lane_key_mask(real, nvalid, g);
      f32x4 s[RB][C::kKT];
      mma_rows<C, RB, !FULL>(s, qcur, koff, kf, km);    // S[q][key] = Q K^T
      sched_phase<RB, C::kKT * C::kDK, 1, 3, 0>();
      __builtin_amdgcn_sched_barrier(0);
      f32x4 lq[C::kKT];
#pragma unroll
      for (int kt = 0; kt < C::kKT; ++kt) lq[kt] = *reinterpret_cast<const f32x4*>(lcur + 16 * kt + 4 * g);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)   // P[q][key]
            s[rb][kt][r] = __builtin_amdgcn_exp2f(fmaf(s[rb][kt][r], p.scale_log2, -lq[kt][r] * kLog2e));
      bf16x8 wf[RB][C::kKP];
      pack_bf16<C, RB>(wf, s);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kp = 0; kp < C::kKP; ++kp) pbuf[pair][rb * C::kKP + kp][lane] = wf[rb][kp];
      __syncthreads();                        // P of this chunk is visible to wave S
      mma_tr<C, RB>(dv, ocur, voff, wf);     // dV^T[d][key] += dO^T P
      sched_phase<RB, C::kKP * C::kDB, 2, 2, 0>();
    };
    for (int it = 0; it < walk.n_chunks; it += 2) {
      step(qb0, ob0, lb0, qb1, ob1, lb1, db1, it);
      if (it + 1 < walk.n_chunks) step(qb1, ob1, lb1, qb0, ob0, lb0, db0, it + 1);
    }
    store_rows<C, RB>(dv, static_cast<bf16_t*>(b.dv) + t.head_base, rm, g, 1.0f);
  } else {
    bf16x8 vf[RB][C::kDK];
    load_frags<C, RB>(vf, vg, rm, g);
    f32x4 dk[RB][C::kDB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) dk[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto step = [&](const char* qcur, const char* ocur, const float* dcur, char* qnxt, char* onxt,
                    float* lnxt, float* dnxt, int it) __attribute__((always_inline)) {
      int row0, nvalid;
      walk.at(it, &row0, &nvalid);
      wait_vm_all();
      __syncthreads();
      if (it + 1 < walk.n_chunks) dma(it + 1, qnxt, onxt, lnxt, dnxt);
      f32x4 dp[RB][C::kKT];
      mma_rows<C, RB>(dp, ocur, koff, vf);   // dP[q][key] = dO V^T
      sched_phase<RB, C::kKT * C::kDK, 1, 3, 0>();
      __builtin_amdgcn_sched_barrier(0);
      f32x4 dq_[C::kKT];
#pragma unroll
      for (int kt = 0; kt < C::kKT; ++kt) dq_[kt] = *reinterpret_cast<const f32x4*>(dcur + 16 * kt + 4 * g);
      __syncthreads();                        // wave P has written this chunk's P
      bf16x8 wd[RB][C::kKP];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kp = 0; kp < C::kKP; ++kp) {
          const bf16x8 pw = pbuf[pair][rb * C::kKP + kp][lane];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            // slot j holds query row 32*kp + 4g + j (j < 4), or + 16 + (j - 4)
            const int kt = 2 * kp + j / 4, r = j % 4;
            wd[rb][kp][j] = static_cast<bf16_t>(static_cast<float>(pw[j]) * (dp[rb][kt][r] - dq_[kt][r]));
          }
        }
      mma_tr<C, RB>(dk, qcur, voff, wd);     // dK^T[d][key] += Q^T dS
      sched_phase<RB, C::kKP * C::kDB, 2, 2, 0>();
    };
    for (int it = 0; it < walk.n_chunks; it += 2) {
      step(qb0, ob0, db0, qb1, ob1, lb1, db1, it);
      if (it + 1 < walk.n_chunks) step(qb1, ob1, db1, qb0, ob0, lb0, db0, it + 1);
    }
    store_rows<C, RB>(dk, static_cast<bf16_t*>(b.dk) + t.head_base, rm, g, b.scale);
  }
}

// ---------------------------------------------------------------------------
// f32 kernels: 32 own rows an item, two lanes a row, the walk split over waves
// ---------------------------------------------------------------------------
// As the float32 forward: lane l keeps dimensions D/2 * (l / 32) .. of own
// row l % 32 (a dot product is the sum of the two halves, exchanged by a
// permlane swap); the walk's 32-row chunks are dealt to the KS waves of the
// workgroup in turn (wave w takes chunks w, w + KS, ...), each staged in the
// wave's own LDS buffers with no workgroup barrier; no softmax state is
// carried (P comes from lse), so the waves' partial gradients simply add up
// through LDS at the end, in a fixed order.

// Rows of chunk c of the walk (32 rows of run c / cpr) into this wave's two
// buffers: a and b rows (K and V, or Q and dO) as float4, zero past the run.
template <int D, bool RASTER>
__device__ __forceinline__ void f32_stage_chunk(const AttnParams& p, const KvRuns& kv, int run, int c0,
                                                int nvalid, const float4* ga, const float4* gb,
                                                float4* la, float4* lb, int lane) {
  constexpr int D4 = D / 4;
  constexpr int kPer = kF32BN * D4 / 64;   // float4 of each operand per lane
  constexpr int kGroup = D <= 64 ? (kPer < 8 ? kPer : 8) : 4;
  const int row0 = RASTER ? kv.run_start_raster(run, p.H, p.W, p.ct, p.ch, p.cw) : kv.run_start(run);
#pragma unroll
  for (int r0 = 0; r0 < kPer; r0 += kGroup) {
    float4 xa[kGroup], xb[kGroup];
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
      const int i = lane + 64 * (r0 + r);
      const int key = i / D4;
      xa[r] = xb[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (key < nvalid) {
        const int tok = row0 + (RASTER ? run_offset_raster(p, c0 + key) : c0 + key);
        const long long off = (long long)tok * D4 + (i - key * D4);
        xa[r] = ga[off];
        xb[r] = gb[off];
      }
    }
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
      la[lane + 64 * (r0 + r)] = xa[r];
      lb[lane + 64 * (r0 + r)] = xb[r];
    }
  }
}

// Token of chunk row `key` (< nvalid) of run `run` of the walk.
template <bool RASTER>
__device__ __forceinline__ int f32_walk_token(const AttnParams& p, const KvRuns& kv, int run, int e) {
  return RASTER ? kv.run_start_raster(run, p.H, p.W, p.ct, p.ch, p.cw) + run_offset_raster(p, e)
                : kv.run_start(run) + e;
}

// Half-row dot product: this lane's DH dimensions against row j of a staged
// chunk (its half), summed with the partner lane's half.
template <int D>
__device__ __forceinline__ float f32_row_dot(const float (&x)[D / 2], const float4* rows, int j) {
  constexpr int D4 = D / 4;
  float acc = 0.f;
#pragma unroll
  for (int d4 = 0; d4 < D4 / 2; ++d4) {
    const float4 y = rows[j * D4 + d4];
    acc = fmaf(x[4 * d4], y.x, acc);
    acc = fmaf(x[4 * d4 + 1], y.y, acc);
    acc = fmaf(x[4 * d4 + 2], y.z, acc);
    acc = fmaf(x[4 * d4 + 3], y.w, acc);
  }
  return pair32(acc, false);
}

template <int D>
__device__ __forceinline__ void f32_row_axpy(float (&acc)[D / 2], float a, const float4* rows, int j) {
  constexpr int D4 = D / 4;
#pragma unroll
  for (int d4 = 0; d4 < D4 / 2; ++d4) {
    const float4 y = rows[j * D4 + d4];
    acc[4 * d4] = fmaf(a, y.x, acc[4 * d4]);
    acc[4 * d4 + 1] = fmaf(a, y.y, acc[4 * d4 + 1]);
    acc[4 * d4 + 2] = fmaf(a, y.z, acc[4 * d4 + 2]);
    acc[4 * d4 + 3] = fmaf(a, y.w, acc[4 * d4 + 3]);
  }
}

// Own-row token of lane row `row` (row 0 of the item when the row does not
// exist: read, never written).
template <bool RASTER>
__device__ __forceinline__ int f32_own_token(const AttnParams& p, const Task& t, int row) {
  const int r = row < t.valid_rows ? row : 0;
  return RASTER ? tile_row_raster(p, t.qt, t.qh, t.qw, t.local0 + r) : t.row0 + r;
}

// dQ: own rows are queries, the walk is the window's keys.
template <int D, bool RASTER>
__global__ void __launch_bounds__(f32_key_splits(D) * 64) bwd_f32_dq_kernel(const AttnParams p, const BwdParams b) {
  constexpr int KS = f32_key_splits(D);
  constexpr int D4 = D / 4;
  constexpr int DH = D / 2;
  constexpr int R = kF32Rows;
  constexpr int kStage = KS * 2 * kF32BN * D4;
  constexpr int kMerge = KS * D * R / 4;
  __shared__ float4 lds[kStage > kMerge ? kStage : kMerge];
  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<R>(p, task, D);
  const long long rowbase = t.head_base / D;
  const float* qg = static_cast<const float*>(p.q) + t.head_base;
  const float4* kg = reinterpret_cast<const float4*>(static_cast<const float*>(p.k) + t.head_base);
  const float4* vg = reinterpret_cast<const float4*>(static_cast<const float*>(p.v) + t.head_base);
  const float* dog = static_cast<const float*>(b.dout) + t.head_base;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & (R - 1);
  const int half = lane / R;
  const int tok = f32_own_token<RASTER>(p, t, row);
  float q[DH], d_o[DH], acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    q[d] = qg[(long long)tok * D + half * DH + d];
    d_o[d] = dog[(long long)tok * D + half * DH + d];
    acc[d] = 0.f;
  }
  const float lse2 = b.lse[rowbase + tok] * kLog2e;
  const float dl = b.delta[rowbase + tok];
  float4* ks = lds + wave * (2 * kF32BN * D4);
  float4* vs = ks + kF32BN * D4;
  const int cpr = (t.kv.run_len + kF32BN - 1) / kF32BN;
  const int n_chunks = t.kv.runs * cpr;
  for (int c = wave; c < n_chunks; c += KS) {
    const int run = c / cpr;
    const int c0 = (c - run * cpr) * kF32BN;
    const int nvalid = min(kF32BN, t.kv.run_len - c0);
    f32_stage_chunk<D, RASTER>(p, t.kv, run, c0, nvalid, kg, vg, ks, vs, lane);
    const float4* kh = ks + half * (D4 / 2);
    const float4* vh = vs + half * (D4 / 2);
#pragma unroll 1
    for (int j = 0; j < kF32BN; ++j) {
      const float sq = f32_row_dot<D>(q, kh, j);
      const float sp = f32_row_dot<D>(d_o, vh, j);
      const float pr = j < nvalid ? __builtin_amdgcn_exp2f(fmaf(sq, p.scale_log2, -lse2)) : 0.f;
      f32_row_axpy<D>(acc, pr * (sp - dl), kh, j);
    }
  }
  __syncthreads();   // every wave is done with its chunk buffers
  float* ob = reinterpret_cast<float*>(lds);   // [KS][D][R]
#pragma unroll
  for (int d = 0; d < DH; ++d) ob[(wave * D + half * DH + d) * R + row] = acc[d];
  __syncthreads();
  if (row < t.valid_rows) {
    float* dst = static_cast<float*>(b.dq) + t.head_base + (long long)tok * D;
    constexpr int kDims = D / KS / 2;
#pragma unroll
    for (int dd = 0; dd < kDims; ++dd) {
      const int d = (2 * wave + half) * kDims + dd;
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < KS; ++w) x += ob[(w * D + d) * R + row];
      dst[d] = x * b.scale;
    }
  }
}

// dK, dV: own rows are keys, the walk is the query rows of the query tiles
// whose window holds the key tile.
template <int D, bool RASTER>
__global__ void __launch_bounds__(f32_key_splits(D) * 64) bwd_f32_dkdv_kernel(const AttnParams p, const BwdParams b) {
  constexpr int KS = f32_key_splits(D);
  constexpr int D4 = D / 4;
  constexpr int DH = D / 2;
  constexpr int R = kF32Rows;
  constexpr int kStage = KS * 2 * kF32BN * D4;
  constexpr int kMerge = KS * 2 * D * R / 4;   // dK and dV
  __shared__ float4 lds[kStage > kMerge ? kStage : kMerge];
  __shared__ float lsb[KS][kF32BN];   // the chunk's lse (base 2) and D
  __shared__ float dsb[KS][kF32BN];
  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<R, true>(p, task, D);
  const long long rowbase = t.head_base / D;
  const float4* qg = reinterpret_cast<const float4*>(static_cast<const float*>(p.q) + t.head_base);
  const float* kg = static_cast<const float*>(p.k) + t.head_base;
  const float* vg = static_cast<const float*>(p.v) + t.head_base;
  const float4* dog = reinterpret_cast<const float4*>(static_cast<const float*>(b.dout) + t.head_base);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & (R - 1);
  const int half = lane / R;
  const int tok = f32_own_token<RASTER>(p, t, row);
  float k[DH], v[DH], dk[DH], dv[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    k[d] = kg[(long long)tok * D + half * DH + d];
    v[d] = vg[(long long)tok * D + half * DH + d];
    dk[d] = dv[d] = 0.f;
  }
  float4* qs = lds + wave * (2 * kF32BN * D4);
  float4* os = qs + kF32BN * D4;
  const int cpr = (t.kv.run_len + kF32BN - 1) / kF32BN;
  const int n_chunks = t.kv.runs * cpr;
  for (int c = wave; c < n_chunks; c += KS) {
    const int run = c / cpr;
    const int c0 = (c - run * cpr) * kF32BN;
    const int nvalid = min(kF32BN, t.kv.run_len - c0);
    f32_stage_chunk<D, RASTER>(p, t.kv, run, c0, nvalid, qg, dog, qs, os, lane);
    if (lane < kF32BN) {
      float l2 = 0.f, dd = 0.f;
      if (lane < nvalid) {
        const int qt = f32_walk_token<RASTER>(p, t.kv, run, c0 + lane);
        l2 = b.lse[rowbase + qt] * kLog2e;
        dd = b.delta[rowbase + qt];
      }
      lsb[wave][lane] = l2;
      dsb[wave][lane] = dd;
    }
    const float4* qh = qs + half * (D4 / 2);
    const float4* oh = os + half * (D4 / 2);
#pragma unroll 1
    for (int j = 0; j < kF32BN; ++j) {
      const float sq = f32_row_dot<D>(k, qh, j);
      const float sp = f32_row_dot<D>(v, oh, j);
      const float pr = j < nvalid ? __builtin_amdgcn_exp2f(fmaf(sq, p.scale_log2, -lsb[wave][j])) : 0.f;
      f32_row_axpy<D>(dv, pr, oh, j);
      f32_row_axpy<D>(dk, pr * (sp - dsb[wave][j]), qh, j);
    }
  }
  __syncthreads();   // every wave is done with its chunk buffers
  float* ob = reinterpret_cast<float*>(lds);   // [KS][2][D][R]: dK, then dV
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    ob[((wave * 2 + 0) * D + half * DH + d) * R + row] = dk[d];
    ob[((wave * 2 + 1) * D + half * DH + d) * R + row] = dv[d];
  }
  __syncthreads();
  if (row < t.valid_rows) {
    float* dkd = static_cast<float*>(b.dk) + t.head_base + (long long)tok * D;
    float* dvd = static_cast<float*>(b.dv) + t.head_base + (long long)tok * D;
    constexpr int kDims = D / KS / 2;
#pragma unroll
    for (int dd = 0; dd < kDims; ++dd) {
      const int d = (2 * wave + half) * kDims + dd;
      float xk = 0.f, xv = 0.f;
#pragma unroll
      for (int w = 0; w < KS; ++w) {
        xk += ob[((w * 2 + 0) * D + d) * R + row];
        xv += ob[((w * 2 + 1) * D + d) * R + row];
      }
      dkd[d] = xk * b.scale;
      dvd[d] = xv;
    }
  }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------


// LDS for the raster offsets of the longest run: omega_w * tau keys for the
// query side, the longest transposed interval along w times tau for the key
// side.
unsigned raster_bytes(const AttnProblem& a, bool keys) {
  int run = 0;
  for (int h = 0; h < a.heads; ++h) {
    int len = a.omega[h][2];
    if (keys) {
      len = 0;
      for (int j = 0; j < a.g.nw; ++j) {
        int lo, hi;
        window_inverse(j, a.g.nw, a.omega[h][2], &lo, &hi);
        len = hi - lo + 1 > len ? hi - lo + 1 : len;
      }
    }
    run = len * a.g.tau > run ? len * a.g.tau : run;
  }
  return (unsigned)run * sizeof(int);
}

template <int D, int WAVES, int RB, bool KEYS, bool PAD, bool FULL>
void launch_pass_kernel(const AttnParams& p, const BwdParams& b, unsigned grid, bool raster,
                        unsigned lds, hipStream_t stream) {
  using C = Bf16Cfg<D, WAVES, RB, 64>;
  if constexpr (KEYS) {
    if (raster)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, WAVES, RB, 64, true, PAD, FULL>), dim3(grid), dim3(C::kThreads), lds, stream, p, b);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, WAVES, RB, 64, false, PAD, FULL>), dim3(grid), dim3(C::kThreads), 0, stream, p, b);
  } else {
    if (raster)
      hipLaunchKernelGGL((bwd_dq_kernel<D, WAVES, RB, 64, true, PAD, FULL>), dim3(grid), dim3(C::kThreads), lds, stream, p, b);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, WAVES, RB, 64, false, PAD, FULL>), dim3(grid), dim3(C::kThreads), 0, stream, p, b);
  }
}

template <int D, int WAVES, int RB, bool KEYS>
int launch_bf16_pass(const BwdProblem& pr, hipStream_t stream) {
  using C = Bf16Cfg<D, WAVES, RB, 64>;
  AttnParams p;
  BwdParams b;
  fill_bwd_params(pr, C::kRows, &p, &b);
  const unsigned grid = (unsigned)p.per_xcd * kXcds;
  const bool raster = pr.attn.raster;
  const unsigned lds = raster ? raster_bytes(pr.attn, KEYS) : 0;
  // Whole 64-row chunks everywhere (every run is a whole number of tiles):
  // no chunk needs masking.
  if (pr.attn.g.padded)
    launch_pass_kernel<D, WAVES, RB, KEYS, true, false>(p, b, grid, raster, lds, stream);
  else if (pr.attn.g.tau % 64 == 0)
    launch_pass_kernel<D, WAVES, RB, KEYS, false, true>(p, b, grid, raster, lds, stream);
  else
    launch_pass_kernel<D, WAVES, RB, KEYS, false, false>(p, b, grid, raster, lds, stream);
  return (int)hipGetLastError();
}

// Key side with paired waves: PAIRS pairs of 16 * RB key rows. Sharing more
// key rows a pair cuts the LDS bytes each MFMA needs (every streamed
// fragment feeds RB products): 48 rows a pair measured 6-8 % faster than 32
// on the 30x48x80 workloads, bit-identical gradients. Rows that are not
// tokens are handled by -inf starts, not selects, which keeps every variant
// within the registers.
template <int D, int PAIRS, int RB>
int launch_bf16_pair_pass(const BwdProblem& pr, hipStream_t stream) {
  constexpr int kThreads = 2 * PAIRS * 64;
  AttnParams p;
  BwdParams b;
  fill_bwd_params(pr, PAIRS * 16 * RB, &p, &b);
  const unsigned grid = (unsigned)p.per_xcd * kXcds;
  const bool raster = pr.attn.raster;
  const unsigned lds = raster ? raster_bytes(pr.attn, true) : 0;
  if (pr.attn.g.padded) {
    if (raster)
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, PAIRS, RB, 64, true, true, false>), dim3(grid), dim3(kThreads), lds, stream, p, b);
    else
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, PAIRS, RB, 64, false, true, false>), dim3(grid), dim3(kThreads), 0, stream, p, b);
  } else if (pr.attn.g.tau % 64 == 0) {
    if (raster)
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, PAIRS, RB, 64, true, false, true>), dim3(grid), dim3(kThreads), lds, stream, p, b);
    else
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, PAIRS, RB, 64, false, false, true>), dim3(grid), dim3(kThreads), 0, stream, p, b);
  } else {
    if (raster)
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, PAIRS, RB, 64, true, false, false>), dim3(grid), dim3(kThreads), lds, stream, p, b);
    else
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, PAIRS, RB, 64, false, false, false>), dim3(grid), dim3(kThreads), 0, stream, p, b);
  }
  return (int)hipGetLastError();
}

template <int D>
int launch_bf16_bwd(const BwdProblem& pr, hipStream_t stream) {
  // Key side: pairs of waves sharing 32 key rows (or 16 key rows per wave on
  // small tiles); query side: 32 query rows per wave.
  const int tau = pr.attn.g.tau;
  const int kr = bwd_key_rows(tau);
  int rc = kr == 192   ? launch_bf16_pair_pass<D, 4, 3>(pr, stream)
           : kr == 128 ? launch_bf16_pair_pass<D, 4, 2>(pr, stream)
                       : launch_bf16_pass<D, 4, 1, true>(pr, stream);
  if (rc) return rc;
  return bwd_query_rows(tau) == 128 ? launch_bf16_pass<D, 4, 2, false>(pr, stream)
                                    : launch_bf16_pass<D, 4, 1, false>(pr, stream);
}

template <int D>
int launch_f32_bwd(const BwdProblem& pr, hipStream_t stream) {
  AttnParams p;
  BwdParams b;
  fill_bwd_params(pr, kF32Rows, &p, &b);
  const unsigned grid = (unsigned)p.per_xcd * kXcds;
  constexpr int kThreads = f32_key_splits(D) * 64;
  if (pr.attn.raster) {
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, true>), dim3(grid), dim3(kThreads), 0, stream, p, b);
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, true>), dim3(grid), dim3(kThreads), 0, stream, p, b);
  } else {
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, false>), dim3(grid), dim3(kThreads), 0, stream, p, b);
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, false>), dim3(grid), dim3(kThreads), 0, stream, p, b);
  }
  return (int)hipGetLastError();
}

template <typename T, int D>
int launch_delta(const BwdProblem& pr, hipStream_t stream) {
  const AttnProblem& a = pr.attn;
  const long long rows = (long long)a.B * a.heads * (a.raster ? a.g.S : a.g.S_pad);
  const long long chunks = rows * (D / (16 / (int)sizeof(T)));
  const unsigned grid = (unsigned)((chunks + 255) / 256);
  hipLaunchKernelGGL((delta_kernel<T, D>), dim3(grid), dim3(256), 0, stream,
                     static_cast<const T*>(a.out), static_cast<const T*>(pr.dout), pr.delta, rows);
  return (int)hipGetLastError();
}

}  // namespace

int launch_backward(const BwdProblem& pr, void* stream_ptr) {
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const AttnProblem& a = pr.attn;
  const long long tasks_upper = (long long)a.B * a.heads * a.g.n_tiles * a.g.tau;
  if (tasks_upper > (1LL << 31) - 1) return (int)hipErrorInvalidValue;
  int rc;
  if (a.dtype == STA_BF16) {
    if (a.head_dim == 128) {
      if ((rc = launch_delta<bf16_t, 128>(pr, stream))) return rc;
      return launch_bf16_bwd<128>(pr, stream);
    }
    if (a.head_dim == 64) {
      if ((rc = launch_delta<bf16_t, 64>(pr, stream))) return rc;
      return launch_bf16_bwd<64>(pr, stream);
    }
  } else if (a.dtype == STA_F32) {
    if (a.head_dim == 128) {
      if ((rc = launch_delta<float, 128>(pr, stream))) return rc;
      return launch_f32_bwd<128>(pr, stream);
    }
    if (a.head_dim == 64) {
      if ((rc = launch_delta<float, 64>(pr, stream))) return rc;
      return launch_f32_bwd<64>(pr, stream);
    }
  }
  return STA_ERR_UNSUPPORTED;
}

}  // namespace sta
