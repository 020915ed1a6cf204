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
// f32 kernels (float32 problems): one wavefront per own row, the head
// dimension split over the lanes, dot products reduced across the wave.
#include <hip/hip_runtime.h>

#include "sta_attn_common.h"

namespace sta {
namespace {

struct BwdParams {
  const void* dout;    // dO, same shape and order as q
  const float* lse;    // [B][heads][S] forward log-sum-exp (natural log)
  float* delta;        // [B][heads][S] D = dO . O (written by delta_kernel)
  void* dq;
  void* dk;
  void* dv;
  float scale;
};

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
// 16*kt + 4g + r against own row l16 of block rb.
template <class C, int RB>
__device__ __forceinline__ void mma_rows(f32x4 (&acc)[RB][C::kKT], const char* buf,
                                         const int (&koff)[C::kDK],
                                         const bf16x8 (&fr)[RB][C::kDK]) {
#pragma unroll
  for (int kt = 0; kt < C::kKT; ++kt) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
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
                                                int lane, const int* rtab, unsigned long long real) {
  const int key = min(lane, nvalid - 1);
  int rel = rtab ? rtab[key] : key;
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
    f32x4 s[RB][C::kKT], dp[RB][C::kKT];
    mma_rows<C, RB>(s, kcur, koff, qf);    // S^T[key][row] = K Q^T
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
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * kt + 4 * g + r;
          const bool off = !FULL && ((nvalid < C::kBN && key >= nvalid) || !((real >> key) & 1ull));
          s[rb][kt][r] = off ? 0.f : s[rb][kt][r] * (dp[rb][kt][r] - dl[rb]);   // dS^T
        }
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
    int base, c0, nv;
    const int* tab = nullptr;
    if (RASTER) {
      walk.at_raster(p, it, &base, &c0, &nv);
      tab = rtab + c0;
    } else {
      walk.at(it, &base, &nv);
    }
    const unsigned long long real = chunk_real_keys<PAD>(p, walk, it, lane);
    load_rows<C, WAVES>(qg, base, nv, qdst, wave, lane, tab, real);
    load_rows<C, WAVES>(dog, base, nv, odst, wave, lane, tab, real);
    if (wave == 0) {
      load_row_values(lseg, base, nv, ldst, lane, tab, real);
      load_row_values(delg, base, nv, ddst, lane, tab, real);
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
    f32x4 s[RB][C::kKT];
    mma_rows<C, RB>(s, qcur, koff, kf);    // S[q][key] = Q K^T
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
        for (int r = 0; r < 4; ++r) {
          const int qrow = 16 * kt + 4 * g + r;
          const bool off = !FULL && ((nvalid < C::kBN && qrow >= nvalid) || !((real >> qrow) & 1ull));
          const float pr = __builtin_amdgcn_exp2f(fmaf(s[rb][kt][r], p.scale_log2, -lq[kt][r] * kLog2e));
          s[rb][kt][r] = off ? 0.f : pr;                  // P[q][key]
        }
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
        for (int r = 0; r < 4; ++r) {
          // a masked row may carry garbage lse / D (padding rows of a tile-major
          // tensor are never written): select, do not multiply
          const int qrow = 16 * kt + 4 * g + r;
          const bool off = !FULL && ((nvalid < C::kBN && qrow >= nvalid) || !((real >> qrow) & 1ull));
          s[rb][kt][r] = off ? 0.f : s[rb][kt][r] * (dp[rb][kt][r] - dq_[kt][r]);   // dS
        }
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
// f32 kernels: one wavefront per own row
// ---------------------------------------------------------------------------

constexpr int kF32Waves = 4;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Own-row token of wave `wave` in the work item (or -1 when it has none).
template <bool RASTER>
__device__ __forceinline__ int own_token(const AttnParams& p, const Task& t, int wave) {
  if (wave >= t.valid_rows) return -1;
  return RASTER ? tile_row_raster(p, t.qt, t.qh, t.qw, t.local0 + wave) : t.row0 + wave;
}

// Token of key (or query) `e` of run `run` of the walk.
template <bool RASTER>
__device__ __forceinline__ int walk_token(const AttnParams& p, const KvRuns& kv, int run, int e) {
  return RASTER ? kv.run_start_raster(run, p.H, p.W, p.ct, p.ch, p.cw) + run_offset_raster(p, e)
                : kv.run_start(run) + e;
}

template <int D, bool RASTER>
__global__ void __launch_bounds__(kF32Waves * 64) bwd_f32_dq_kernel(const AttnParams p, const BwdParams b) {
  constexpr int E = D / 64;
  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<kF32Waves>(p, task, D);
  const int lane = threadIdx.x & 63;
  const int tok = own_token<RASTER>(p, t, threadIdx.x >> 6);
  if (tok < 0) return;
  const long long rowbase = t.head_base / D;
  const float* qg = static_cast<const float*>(p.q) + t.head_base;
  const float* kg = static_cast<const float*>(p.k) + t.head_base;
  const float* vg = static_cast<const float*>(p.v) + t.head_base;
  const float* dog = static_cast<const float*>(b.dout) + t.head_base;
  float q[E], d_o[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = qg[(long long)tok * D + lane + 64 * e];
    d_o[e] = dog[(long long)tok * D + lane + 64 * e];
    acc[e] = 0.f;
  }
  const float lse2 = b.lse[rowbase + tok] * kLog2e;
  const float dl = b.delta[rowbase + tok];
  for (int run = 0; run < t.kv.runs; ++run)
    for (int e = 0; e < t.kv.run_len; ++e) {
      const long long kr = (long long)walk_token<RASTER>(p, t.kv, run, e) * D;
      float sq = 0.f, sp = 0.f;
#pragma unroll
      for (int x = 0; x < E; ++x) {
        sq = fmaf(q[x], kg[kr + lane + 64 * x], sq);
        sp = fmaf(d_o[x], vg[kr + lane + 64 * x], sp);
      }
      const float pr = __builtin_amdgcn_exp2f(fmaf(wave_sum(sq), p.scale_log2, -lse2));
      const float ds = pr * (wave_sum(sp) - dl);
#pragma unroll
      for (int x = 0; x < E; ++x) acc[x] = fmaf(ds, kg[kr + lane + 64 * x], acc[x]);
    }
  float* dqg = static_cast<float*>(b.dq) + t.head_base;
#pragma unroll
  for (int e = 0; e < E; ++e) dqg[(long long)tok * D + lane + 64 * e] = acc[e] * b.scale;
}

template <int D, bool RASTER>
__global__ void __launch_bounds__(kF32Waves * 64) bwd_f32_dkdv_kernel(const AttnParams p, const BwdParams b) {
  constexpr int E = D / 64;
  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<kF32Waves, true>(p, task, D);
  const int lane = threadIdx.x & 63;
  const int tok = own_token<RASTER>(p, t, threadIdx.x >> 6);
  if (tok < 0) return;
  const long long rowbase = t.head_base / D;
  const float* qg = static_cast<const float*>(p.q) + t.head_base;
  const float* kg = static_cast<const float*>(p.k) + t.head_base;
  const float* vg = static_cast<const float*>(p.v) + t.head_base;
  const float* dog = static_cast<const float*>(b.dout) + t.head_base;
  float k[E], v[E], dk[E], dv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = kg[(long long)tok * D + lane + 64 * e];
    v[e] = vg[(long long)tok * D + lane + 64 * e];
    dk[e] = dv[e] = 0.f;
  }
  for (int run = 0; run < t.kv.runs; ++run)
    for (int e = 0; e < t.kv.run_len; ++e) {
      const int qtok = walk_token<RASTER>(p, t.kv, run, e);
      const long long qr = (long long)qtok * D;
      float sq = 0.f, sp = 0.f;
#pragma unroll
      for (int x = 0; x < E; ++x) {
        sq = fmaf(qg[qr + lane + 64 * x], k[x], sq);
        sp = fmaf(dog[qr + lane + 64 * x], v[x], sp);
      }
      const float pr = __builtin_amdgcn_exp2f(
          fmaf(wave_sum(sq), p.scale_log2, -b.lse[rowbase + qtok] * kLog2e));
      const float ds = pr * (wave_sum(sp) - b.delta[rowbase + qtok]);
#pragma unroll
      for (int x = 0; x < E; ++x) {
        dk[x] = fmaf(ds, qg[qr + lane + 64 * x], dk[x]);
        dv[x] = fmaf(pr, dog[qr + lane + 64 * x], dv[x]);
      }
    }
  float* dkg = static_cast<float*>(b.dk) + t.head_base;
  float* dvg = static_cast<float*>(b.dv) + t.head_base;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dkg[(long long)tok * D + lane + 64 * e] = dk[e] * b.scale;
    dvg[(long long)tok * D + lane + 64 * e] = dv[e];
  }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

void fill_bwd_params(const BwdProblem& pr, int rows_per_item, AttnParams* p, BwdParams* b) {
  const AttnProblem& a = pr.attn;
  p->q = a.q; p->k = a.k; p->v = a.v; p->out = a.out;
  p->lse = nullptr;
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

template <int D>
int launch_bf16_bwd(const BwdProblem& pr, hipStream_t stream) {
  // Key side: 16 key rows per wave; query side: 32 query rows per wave.
  int rc = pr.attn.g.tau >= 128 ? launch_bf16_pass<D, 8, 1, true>(pr, stream)
                                : launch_bf16_pass<D, 4, 1, true>(pr, stream);
  if (rc) return rc;
  return pr.attn.g.tau >= 128 ? launch_bf16_pass<D, 4, 2, false>(pr, stream)
                              : launch_bf16_pass<D, 4, 1, false>(pr, stream);
}

template <int D>
int launch_f32_bwd(const BwdProblem& pr, hipStream_t stream) {
  AttnParams p;
  BwdParams b;
  fill_bwd_params(pr, kF32Waves, &p, &b);
  const unsigned grid = (unsigned)p.per_xcd * kXcds;
  if (pr.attn.raster) {
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, true>), dim3(grid), dim3(kF32Waves * 64), 0, stream, p, b);
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, true>), dim3(grid), dim3(kF32Waves * 64), 0, stream, p, b);
  } else {
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, false>), dim3(grid), dim3(kF32Waves * 64), 0, stream, p, b);
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, false>), dim3(grid), dim3(kF32Waves * 64), 0, stream, p, b);
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
