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

#include "sta_kernels.h"

namespace sta {
namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;  // MI355X dispatches workgroups round-robin over 8 XCDs

// Parameters shared by both kernels.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int S;            // tokens per (batch, head)
  int heads;
  int n_tasks;      // work items
  int per_xcd;      // ceil(n_tasks / kXcds)
  int row_blocks;   // work items per query unit
  int n_units;      // query units per (batch, head): tiles, or 1 if dense
  int unit_rows;    // rows per query unit: tau, or S if dense
  float scale_log2; // scale * log2(e)
  int dense;
  int nt, nh, nw, tau;
  uint16_t omega[STA_MAX_HEADS][3];
};

// Maps the hardware workgroup id to a logical task so that consecutive
// logical tasks (the row blocks of one query tile, then neighbouring tiles
// that share most of their keys) run on the same XCD and share its L2.
__device__ __forceinline__ int logical_task(const AttnParams& p) {
  const int bid = blockIdx.x;
  return (bid % kXcds) * p.per_xcd + bid / kXcds;
}

// Key runs of one work item: `runs` runs of `run_len` tokens; run r starts at
// token run_start(r).
struct KvRuns {
  int runs, run_len;
  int oh;             // omega_h (runs per t-step)
  int st, sh, sw;     // window start in tiles
  int nh, nw, tau;
  int dense;
  __device__ __forceinline__ int run_start(int r) const {
    if (dense) return 0;
    const int it = r / oh, ih = r - (r / oh) * oh;
    return (((st + it) * nh + (sh + ih)) * nw + sw) * tau;
  }
};

struct Task {
  long long head_base;  // element offset of this (batch, head)
  int row0;             // first query row (token index) of the work item
  int valid_rows;       // rows of the work item inside its unit
  KvRuns kv;
};

template <int ROWS>
__device__ __forceinline__ Task decode_task(const AttnParams& p, int task, int D) {
  Task t;
  const int rb = task % p.row_blocks;
  const int unit_bh = task / p.row_blocks;
  const int unit = unit_bh % p.n_units;
  const int bh = unit_bh / p.n_units;
  const int h = bh % p.heads;
  t.head_base = (long long)bh * p.S * D;
  const int unit_row0 = unit * p.unit_rows;
  t.row0 = unit_row0 + rb * ROWS;
  t.valid_rows = min(ROWS, p.unit_rows - rb * ROWS);
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
    kv.st = window_start(qt, p.nt, ot);
    kv.sh = window_start(qh, p.nh, oh);
    kv.sw = window_start(qw, p.nw, ow);
    kv.oh = oh;
    kv.runs = ot * oh;
    kv.run_len = ow * p.tau;
  }
  return t;
}

__device__ __forceinline__ float wave_xor_max(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask, 64));
}
__device__ __forceinline__ float wave_xor_sum(float x, int mask) {
  return x + __shfl_xor(x, mask, 64);
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------

template <int D, int WAVES, int RB, int BN>
struct Bf16Cfg {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kRowsWave = 16 * RB;
  static constexpr int kRows = WAVES * kRowsWave;
  static constexpr int kDK = D / 32;            // k-steps of S^T = K Q^T
  static constexpr int kDB = D / 16;            // 16-row blocks of O^T
  static constexpr int kKT = BN / 16;           // 16-key score tiles per chunk
  static constexpr int kKP = BN / 32;           // 32-key steps of O^T += V^T P^T
  static constexpr int kRowBytes = D * 2;       // one key row of K or V
  static constexpr int kCPR = kRowBytes / 16;   // 16-byte chunks per row
  static constexpr int kChunkBytes = BN * kRowBytes;       // K (or V) of one chunk
  static constexpr int kBlocks = kChunkBytes / 1024;       // 1 KB LDS-DMA blocks per chunk
  static constexpr int kBlocksPerWave = kBlocks / WAVES;
  static constexpr int kRowsPerBlock = 1024 / kRowBytes;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(kBlocks % WAVES == 0, "each wave loads whole 1 KB blocks");
};

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Physical byte offset of 16-byte chunk `c` of key row `row` in a K/V buffer.
// Chunks are XOR-swizzled by the row so that the 16 rows read by one MFMA
// operand fetch hit distinct LDS banks.
template <int CPR>
__device__ __forceinline__ int swz(int row, int c) {
  return row * (CPR * 16) + ((c ^ (row % CPR)) << 4);
}

// Issue this wave's direct-to-LDS loads of one K/V chunk: key rows
// kv_row0 .. kv_row0 + BN - 1 of the head (rows past `nvalid` repeat the last
// valid row; their scores are masked). Each instruction fills one 1 KB block.
template <class C>
__device__ __forceinline__ void load_chunk(const bf16_t* kg, const bf16_t* vg, int kv_row0,
                                           int nvalid, char* kbuf, char* vbuf, int wave, int lane) {
#pragma unroll
  for (int b = 0; b < C::kBlocksPerWave; ++b) {
    const int blk = wave * C::kBlocksPerWave + b;
    const int row = blk * C::kRowsPerBlock + lane / C::kCPR;
    const int pos = lane % C::kCPR;
    const int c = pos ^ (row % C::kCPR);
    const int src_row = kv_row0 + min(row, nvalid - 1);
    const long long off = (long long)src_row * (C::kRowBytes / 2) + c * 8;
    __builtin_amdgcn_global_load_lds(kg + off, (lds_void*)(kbuf + blk * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vg + off, (lds_void*)(vbuf + blk * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_vm_all() {
  // vmcnt(0); expcnt and lgkmcnt left at their maxima (not waited on).
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int D, int WAVES, int RB, int BN, bool DENSE>
__global__ void __launch_bounds__(WAVES * 64)
attn_bf16_kernel(const AttnParams p) {
  using C = Bf16Cfg<D, WAVES, RB, BN>;
  // Two buffers, each K then V of one chunk. They are separate objects and the
  // loop below selects them statically, so the compiler can tell the chunk
  // being read apart from the one the LDS DMA is filling and does not wait
  // for the prefetch before reading.
  __shared__ __attribute__((aligned(1024))) char smem0[2 * C::kChunkBytes];
  __shared__ __attribute__((aligned(1024))) char smem1[2 * C::kChunkBytes];

  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  Task t = decode_task<C::kRows>(p, task, D);
  if (DENSE) {
    t.kv.runs = 1;
    t.kv.run_len = p.S;
  }
  const bf16_t* qg = static_cast<const bf16_t*>(p.q) + t.head_base;
  const bf16_t* kg = static_cast<const bf16_t*>(p.k) + t.head_base;
  const bf16_t* vg = static_cast<const bf16_t*>(p.v) + t.head_base;
  bf16_t* og = static_cast<bf16_t*>(p.out) + t.head_base;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;

  const int chunks_per_run = (t.kv.run_len + BN - 1) / BN;
  const int n_chunks = t.kv.runs * chunks_per_run;

  // Chunk `it` covers keys run_start(run) + c0 .. + BN of the head.
  auto chunk_rows = [&](int it, int* row0, int* nvalid) {
    const int run = it / chunks_per_run;
    const int c0 = (it - run * chunks_per_run) * BN;
    *row0 = (DENSE ? 0 : t.kv.run_start(run)) + c0;
    *nvalid = min(BN, t.kv.run_len - c0);
  };

  {
    int row0, nv;
    chunk_rows(0, &row0, &nv);
    load_chunk<C>(kg, vg, row0, nv, smem0, smem0 + C::kChunkBytes, wave, lane);
  }

  // Q rows of this lane: row (within the work item) wave*kRowsWave + 16*rb + l16.
  bf16x8 qf[RB][C::kDK];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wave * C::kRowsWave + 16 * rb + l16;
    const bool ok = r < t.valid_rows;
    const bf16_t* src = qg + (long long)(t.row0 + (ok ? r : 0)) * D + 8 * g;
#pragma unroll
    for (int dk = 0; dk < C::kDK; ++dk) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(src + 32 * dk);
      if (!ok) x = bf16x8{};
      qf[rb][dk] = x;
    }
  }

  f32x4 o[RB][C::kDB];
  float m[RB], lsum[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    lsum[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One chunk: wait for its K/V, start the next chunk's loads into the other
  // buffer, then compute.
  auto chunk_step = [&](const char* cur, char* nxt, int it) __attribute__((always_inline)) {
    int nvalid;
    {
      int row0;
      chunk_rows(it, &row0, &nvalid);
    }
    wait_vm_all();     // this wave's loads of chunk `it` have landed in LDS
    __syncthreads();   // ... and every wave's; chunk it-1's buffer is free
    if (it + 1 < n_chunks) {
      int row0, nv;
      chunk_rows(it + 1, &row0, &nv);
      load_chunk<C>(kg, vg, row0, nv, nxt, nxt + C::kChunkBytes, wave, lane);
    }
    const char* kbuf = cur;
    const char* vbuf = cur + C::kChunkBytes;

    // Scores S^T[key][row] for the wave's rows; lane holds keys 16*kt+4g+r of row l16.
    f32x4 s[RB][C::kKT];
#pragma unroll
    for (int kt = 0; kt < C::kKT; ++kt) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int krow = 16 * kt + l16;
#pragma unroll
      for (int dk = 0; dk < C::kDK; ++dk) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(kbuf + swz<C::kCPR>(krow, 4 * dk + g));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][dk], s[rb][kt], 0, 0, 0);
      }
    }
    if (nvalid < BN) {
#pragma unroll
      for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * kt + 4 * g + r >= nvalid)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[rb][kt][r] = -INFINITY;
    }

    // Online softmax, base 2. The reference max m only moves when a row's
    // chunk max exceeds it by more than 8 (then O and l are rescaled); in
    // between, probabilities stay below 2^8, which fp32 sums and bf16 P hold
    // exactly as well as values below 1.
    float mx[RB];
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float a = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < C::kKT; ++kt)
        a = fmaxf(a, fmaxf(fmaxf(s[rb][kt][0], s[rb][kt][1]), fmaxf(s[rb][kt][2], s[rb][kt][3])));
      a = wave_xor_max(a, 16);
      a = wave_xor_max(a, 32);
      mx[rb] = a * p.scale_log2;
      grow |= mx[rb] > m[rb] + 8.0f;
    }
    if (__any(grow)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float m_new = fmaxf(m[rb], mx[rb]);
        const float alpha = __builtin_amdgcn_exp2f(m[rb] - m_new);
        m[rb] = m_new;
        lsum[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) o[rb][db] *= alpha;
      }
    }
    bf16x8 pf[RB][C::kKP];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < C::kKT; ++kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[rb][kt][r], p.scale_log2, -m[rb]));
          ls += e;
          s[rb][kt][r] = e;
        }
      }
      lsum[rb] += ls;
#pragma unroll
      for (int kp = 0; kp < C::kKP; ++kp) {
        bf16x8 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = static_cast<bf16_t>(s[rb][2 * kp][r]);
          x[4 + r] = static_cast<bf16_t>(s[rb][2 * kp + 1][r]);
        }
        pf[rb][kp] = x;
      }
    }

    // O^T[d][row] += V^T[d][key] P^T[key][row]. Slot j of lane group g maps
    // to key 32*kp + 4g + j (j < 4) or 32*kp + 16 + 4g + (j - 4). The
    // transposing LDS read gives lane i of a 16-lane group element (i % 4) of
    // the 4-element piece addressed by lane 4r + i/4, for r = 0..3: lane s of
    // group g addresses key 32*kp + 4g + s/4, columns 16*db + 4*(s%4) .. +4,
    // so lane i receives V[32*kp + 4g + r][16*db + i], r = 0..3.
    const int s4 = l16 >> 2, sq = l16 & 3;
#pragma unroll
    for (int kp = 0; kp < C::kKP; ++kp) {
      const int vrow_lo = 32 * kp + 4 * g + s4;
      const int vrow_hi = vrow_lo + 16;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
        const int col = 16 * db + 4 * sq;  // element column of this lane's piece
        const int c = col >> 3, half = (col & 7) * 2;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vbuf + swz<C::kCPR>(vrow_lo, c) + half));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vbuf + swz<C::kCPR>(vrow_hi, c) + half));
        const i16x4 both[2] = {lo, hi};
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(both);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rb][kp], o[rb][db], 0, 0, 0);
      }
    }
  };

  for (int it = 0; it < n_chunks; it += 2) {
    chunk_step(smem0, smem1, it);
    if (it + 1 < n_chunks) chunk_step(smem1, smem0, it + 1);
  }

  // Normalise and store: lane holds O[row l16][16*db + 4g + r].
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l = lsum[rb];
    l = wave_xor_sum(l, 16);
    l = wave_xor_sum(l, 32);
    const float inv = 1.0f / l;
    const int r = wave * C::kRowsWave + 16 * rb + l16;
    if (r < t.valid_rows) {
      bf16_t* dst = og + (long long)(t.row0 + r) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = static_cast<bf16_t>(o[rb][db][e] * inv);
        *reinterpret_cast<bf16x4*>(dst + 16 * db) = y;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// f32 kernel
// ---------------------------------------------------------------------------

constexpr int kF32Threads = 128;
constexpr int kF32BN = 32;

template <int D>
__global__ void __launch_bounds__(kF32Threads) attn_f32_kernel(const AttnParams p) {
  __shared__ float4 ks[kF32BN * D / 4];
  __shared__ float4 vs[kF32BN * D / 4];
  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<kF32Threads>(p, task, D);
  const float* qg = static_cast<const float*>(p.q) + t.head_base;
  const float4* kg = reinterpret_cast<const float4*>(static_cast<const float*>(p.k) + t.head_base);
  const float4* vg = reinterpret_cast<const float4*>(static_cast<const float*>(p.v) + t.head_base);
  float* og = static_cast<float*>(p.out) + t.head_base;

  const int tid = threadIdx.x;
  const bool row_ok = tid < t.valid_rows;
  float q[D], o[D];
  const float* qrow = qg + (long long)(t.row0 + (row_ok ? tid : 0)) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = row_ok ? qrow[d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int run = 0; run < t.kv.runs; ++run) {
    const int kv0 = t.kv.run_start(run);
    for (int c0 = 0; c0 < t.kv.run_len; c0 += kF32BN) {
      const int nvalid = min(kF32BN, t.kv.run_len - c0);
      __syncthreads();
      for (int i = tid; i < kF32BN * D / 4; i += kF32Threads) {
        const int key = i / (D / 4);
        float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
        if (key < nvalid) {
          const long long off = (long long)(kv0 + c0) * (D / 4) + i;
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
    float* dst = og + (long long)(t.row0 + tid) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) dst[d] = o[d] * inv;
  }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

void fill_params(const AttnProblem& pr, int rows_per_item, AttnParams* p) {
  p->q = pr.q; p->k = pr.k; p->v = pr.v; p->out = pr.out;
  p->S = pr.g.S;
  p->heads = pr.heads;
  p->dense = pr.dense ? 1 : 0;
  p->scale_log2 = pr.scale * kLog2e;
  if (pr.dense) {
    p->n_units = 1;
    p->unit_rows = pr.g.S;
    p->nt = p->nh = p->nw = 1;
    p->tau = pr.g.S;
  } else {
    p->n_units = pr.g.n_tiles;
    p->unit_rows = pr.g.tau;
    p->nt = pr.g.nt; p->nh = pr.g.nh; p->nw = pr.g.nw;
    p->tau = pr.g.tau;
    for (int h = 0; h < pr.heads; ++h)
      for (int a = 0; a < 3; ++a) p->omega[h][a] = pr.omega[h][a];
  }
  p->row_blocks = (p->unit_rows + rows_per_item - 1) / rows_per_item;
  const long long tasks = (long long)pr.B * pr.heads * p->n_units * p->row_blocks;
  p->n_tasks = (int)tasks;
  p->per_xcd = (int)((tasks + kXcds - 1) / kXcds);
}

template <int D, int WAVES, int RB, int BN>
int launch_bf16(const AttnProblem& pr, hipStream_t stream) {
  using C = Bf16Cfg<D, WAVES, RB, BN>;
  AttnParams p;
  fill_params(pr, C::kRows, &p);
  const unsigned grid = (unsigned)p.per_xcd * kXcds;
  if (pr.dense)
    hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, true>), dim3(grid), dim3(C::kThreads),
                       0, stream, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN, false>), dim3(grid), dim3(C::kThreads),
                       0, stream, p);
  return (int)hipGetLastError();
}

template <int D>
int launch_f32(const AttnProblem& pr, hipStream_t stream) {
  AttnParams p;
  fill_params(pr, kF32Threads, &p);
  const unsigned grid = (unsigned)p.per_xcd * kXcds;
  hipLaunchKernelGGL((attn_f32_kernel<D>), dim3(grid), dim3(kF32Threads), 0, stream, p);
  return (int)hipGetLastError();
}

// Rows per bf16 work item: a whole 384-token tile when it fits, else 64 or 128.
template <int D>
int dispatch_bf16(const AttnProblem& pr, hipStream_t stream) {
  const int unit_rows = pr.dense ? pr.g.S : pr.g.tau;
  if (unit_rows % 384 == 0) return launch_bf16<D, 8, 3, 64>(pr, stream);
  if (unit_rows <= 64) return launch_bf16<D, 4, 1, 64>(pr, stream);
  return launch_bf16<D, 4, 2, 64>(pr, stream);
}

}  // namespace

int launch_attention(const AttnProblem& pr, void* stream_ptr) {
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const long long units = pr.dense ? 1 : pr.g.n_tiles;
  const long long tasks_upper = (long long)pr.B * pr.heads * units * (pr.dense ? pr.g.S : pr.g.tau);
  if (tasks_upper > (1LL << 31) - 1) return (int)hipErrorInvalidValue;
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
