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
  static constexpr int kDK = D / 32;     // k-steps of S^T = K Q^T
  static constexpr int kDB = D / 16;     // 16-row blocks of O^T
  static constexpr int kKT = BN / 16;    // 16-key score tiles per chunk
  static constexpr int kKP = BN / 32;    // 32-key steps of O^T += V^T P^T
  static constexpr int kKPitch = D + 8;  // LDS row pitch of K (elements)
  static constexpr int kVPitch = BN + 8; // LDS row pitch of V^T (elements)
  static constexpr int kPieces = BN * D / 8;  // 16-byte pieces per chunk of K (or V)
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
};

template <int D, int WAVES, int RB, int BN>
__global__ void __launch_bounds__(WAVES * 64)
attn_bf16_kernel(const AttnParams p) {
  using C = Bf16Cfg<D, WAVES, RB, BN>;
  __shared__ bf16_t ks[BN * C::kKPitch];
  __shared__ bf16_t vt[D * C::kVPitch];

  const int task = logical_task(p);
  if (task >= p.n_tasks) return;
  const Task t = decode_task<C::kRows>(p, task, D);
  const bf16_t* qg = static_cast<const bf16_t*>(p.q) + t.head_base;
  const bf16_t* kg = static_cast<const bf16_t*>(p.k) + t.head_base;
  const bf16_t* vg = static_cast<const bf16_t*>(p.v) + t.head_base;
  bf16_t* og = static_cast<bf16_t*>(p.out) + t.head_base;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;

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

  for (int run = 0; run < t.kv.runs; ++run) {
    const int kv0 = t.kv.run_start(run);
    for (int c0 = 0; c0 < t.kv.run_len; c0 += BN) {
      const int nvalid = min(BN, t.kv.run_len - c0);
      __syncthreads();  // the previous chunk is no longer read
      // Stage K (row-major) and V (transposed) for keys kv0+c0 .. +BN.
#pragma unroll
      for (int i = tid; i < C::kPieces; i += C::kThreads) {
        const int key = i / (D / 8);
        const int col = (i % (D / 8)) * 8;
        bf16x8 kx = bf16x8{}, vx = bf16x8{};
        if (key < nvalid) {
          const long long off = (long long)(kv0 + c0 + key) * D + col;
          kx = *reinterpret_cast<const bf16x8*>(kg + off);
          vx = *reinterpret_cast<const bf16x8*>(vg + off);
        }
        *reinterpret_cast<bf16x8*>(&ks[key * C::kKPitch + col]) = kx;
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[(col + e) * C::kVPitch + key] = vx[e];
      }
      __syncthreads();

      // Scores S^T[key][row] for the wave's rows; lane holds keys 16*kt+4g+r of row l16.
      f32x4 s[RB][C::kKT];
#pragma unroll
      for (int kt = 0; kt < C::kKT; ++kt) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dk = 0; dk < C::kDK; ++dk) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(&ks[(16 * kt + l16) * C::kKPitch + 32 * dk + 8 * g]);
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

      // Online softmax (base 2) and P in bf16 as the B operand of O^T += V^T P^T.
      bf16x8 pf[RB][C::kKP];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[rb][kt][r]);
        mx = wave_xor_max(mx, 16);
        mx = wave_xor_max(mx, 32);
        const float m_new = fmaxf(m[rb], mx * p.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m[rb] - m_new);
        m[rb] = m_new;
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < C::kKT; ++kt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(s[rb][kt][r] * p.scale_log2 - m_new);
            ls += e;
            s[rb][kt][r] = e;
          }
        }
        lsum[rb] = lsum[rb] * alpha + ls;
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) o[rb][db] *= alpha;
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
      // to key 32*kp + 4g + j (j < 4) or 32*kp + 16 + 4g + (j - 4).
#pragma unroll
      for (int kp = 0; kp < C::kKP; ++kp) {
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) {
          const bf16_t* vrow = &vt[(16 * db + l16) * C::kVPitch + 32 * kp + 4 * g];
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 16);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rb][kp], o[rb][db], 0, 0, 0);
        }
      }
    }
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
  hipLaunchKernelGGL((attn_bf16_kernel<D, WAVES, RB, BN>), dim3(grid), dim3(C::kThreads), 0,
                     stream, p);
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
