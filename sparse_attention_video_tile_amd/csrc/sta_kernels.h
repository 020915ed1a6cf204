// Launch interface between the C-ABI layer (sta_api.cpp) and the HIP kernels.
// Every launcher enqueues on the given stream and returns 0 on success or the
// hipError_t value reported by the runtime right after the launch.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "sta.h"
#include "sta_geometry.h"

namespace sta {

// Largest window run, omega_w * tau keys, the raster-order attention handles
// (the run's table of raster offsets is kept in LDS).
constexpr int kMaxRasterRun = 8192;

// Candidate windows one window-recall pass scores at once, and the largest
// per-chunk candidate table (bytes of dynamic LDS, one per 64-key chunk of
// the whole volume) it keeps.
constexpr int kMaxRecallCand = 8;
constexpr int kMaxRecallTable = 65536;

struct AttnProblem {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;      // optional [B][heads][S] log-sum-exp per query row (natural log)
  int B, heads, head_dim;
  int dtype;       // sta_dtype
  float scale;
  bool dense;      // true: every query attends to all S keys
  bool raster;     // STA only: q, k, v, out in raster order (else tile-major)
  bool lse_only;   // write lse only (out and v are not touched)
  bool qk_fp8;     // q and k are fp8 e4m3 (v and out keep dtype, which is bf16)
  Geometry g;      // for dense problems only g.S is used
  // Window per head in tiles (sparse problems only).
  uint16_t omega[STA_MAX_HEADS][3];
  // Window recall in one pass (lse_only, the whole volume as every head's
  // window): the log-sum-exp of each query row over the keys of candidate
  // window c (in tiles) goes to lse_cand + c * cand_stride, in lse's layout.
  // n_cand = 0 otherwise.
  int n_cand;
  float* lse_cand;
  long long cand_stride;
  uint16_t cand_omega[kMaxRecallCand][3];
};

int launch_reorder(const void* src, void* dst, int BH, int row_bytes, const Geometry& g,
                   bool to_tiles, void* stream);

// transposed: list, per key tile, the query tiles whose window holds it.
int launch_kv_tiles(int* kv_list, int* kv_count, int heads, const Geometry& g,
                    const uint16_t (*omega)[3], int max_kv, bool transposed, void* stream);

// Returns STA_ERR_UNSUPPORTED (as a negative value) when no kernel exists for
// the (dtype, head_dim) pair, 0 on success, or a positive hipError_t.
int launch_attention(const AttnProblem& p, void* stream);

// Gradients of STA (sparse problems only). attn.out holds the forward output
// O; delta is a [B][heads][S] float workspace the launch fills with
// rowsum(dO * O) before the gradient kernels read it.
struct BwdProblem {
  AttnProblem attn;
  const void* dout;
  const float* lse;
  float* delta;
  void* dq;
  void* dk;
  void* dv;
};

// Same return convention as launch_attention.
int launch_backward(const BwdProblem& p, void* stream);

// recall[bh * n_cand + c] = mean over the S rows of exp(lse_win - lse_full),
// for bh < BH (both lse arrays [BH][S]).
int launch_recall_reduce(const float* lse_full, const float* lse_win, float* recall, int BH, int S,
                         int n_cand, int c, void* stream);

// Floats in the device scratch of the allocation-free backward (32 MiB per
// GPU): the D workspace of up to 8 Mi query rows (B * heads * rows).
constexpr long long kNoAllocScratchFloats = 8LL << 20;

// The current device's address of that scratch, looked up on the first call
// on each device. Returns 0 or a hipError_t value.
int noalloc_scratch(float** ptr);

const char* hip_error_string(int code);

}  // namespace sta
