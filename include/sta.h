/*
 * libsta -- Sliding Tile Attention (STA) forward and backward for AMD MI355X
 * (gfx950).
 *
 * STA ("Fast Video Generation with Sliding Tile Attention") replaces full 3D
 * attention over a (T, H, W) latent video. The token grid is cut into tiles of
 * (c_t, c_h, c_w) tokens; the attention window slides tile by tile, so every
 * query of one tile attends to exactly the keys of the tiles inside that
 * tile's 3D window (podcast transcript on hotaipapers.com, the answers on what
 * a tile is and on dense / empty / mixed blocks; dianyo ICML2025 blog, STA
 * "Observation & Proposed Method"). Every (query tile, key tile) block is then
 * either computed densely or skipped; no block is partly masked.
 *
 * Window rule (the pages do not spell it out; this is the reading the library
 * implements): per head a window of w = (w_t, w_h, w_w) tokens, a whole number
 * of tiles per axis, omega_a = w_a / c_a. For a query tile with tile
 * coordinate q_a on an axis of n_a tiles,
 *     start_a = min(max(q_a - omega_a / 2, 0), n_a - omega_a)      (integer /)
 * and the window covers key tiles start_a .. start_a + omega_a - 1. The window
 * keeps its full size at the volume's border (its centre is clamped inside the
 * volume), so each query tile sees exactly omega_t * omega_h * omega_w tiles.
 *
 * Token orders.
 *   raster:     s  = (t * H + y) * W + x
 *   tile-major: s' = tile * tau + local, tau = c_t * c_h * c_w,
 *               tile  = (floor(t/c_t) * n_h + floor(y/c_h)) * n_w + floor(x/c_w),
 *               local = ((t % c_t) * c_h + (y % c_h)) * c_w + (x % c_w)
 *   with n_a = ceil(extent_a / c_a). Tensors are [B][heads][rows][head_dim],
 *   contiguous, in one of these orders as each call states: raster tensors
 *   have S = T * H * W rows, tile-major tensors n_tiles * tau rows.
 *
 * Volumes the tile does not divide (a reading; the pages do not describe
 * padding): the tile grid covers the volume padded up to whole tiles, windows
 * are counted in tiles of that grid with the same rule, and positions past
 * the volume are not tokens -- they are never keys and have no output. In
 * tile-major order they are rows of zeros (sta_reorder_tiles writes zeros,
 * the attention calls leave output rows of padding unwritten). Float32
 * attention on such a volume is refused (STA_ERR_UNSUPPORTED); the layout
 * calls accept it.
 *
 * Conventions for every call.
 *   - Device pointers are caller-owned device memory (e.g. torch tensors). The
 *     library allocates no device memory and keeps no state between calls
 *     apart from a thread-local error message.
 *   - Host arrays (tile, window) are read during the call only; the window
 *     table is copied into the kernel arguments, so it may be freed on return.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     is asynchronous: inputs must stay alive and unmodified until the stream
 *     has passed the work.
 *   - Arguments are validated before anything is enqueued. On any error the
 *     call returns a negative sta_status, enqueues nothing (except STA_ERR_HIP,
 *     which reports a failed launch) and sta_last_error() describes it.
 *   - Outputs must not overlap any input.
 */
#ifndef STA_H_
#define STA_H_

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STA_OK = 0,
  STA_ERR_INVALID_ARG = -1, /* NULL pointer, bad size, tile/window mismatch, overlap */
  STA_ERR_UNSUPPORTED = -2, /* a valid request that no compiled kernel serves */
  STA_ERR_HIP = -3          /* the HIP runtime reported an error at launch */
} sta_status;

typedef enum {
  STA_BF16 = 0, /* bfloat16 storage, float32 accumulation */
  STA_F32 = 1   /* float32 storage and arithmetic */
} sta_dtype;

typedef enum {
  STA_TILE_MAJOR = 0, /* tensors in tile-major token order */
  STA_RASTER = 1      /* tensors in raster token order */
} sta_order;

/* Largest head count whose window table fits the kernel arguments. */
#define STA_MAX_HEADS 256

/* Version of this interface; bumped on any incompatible change. */
int sta_abi_version(void);

/*
 * Permute the token axis from raster to tile-major order (a bit-exact copy).
 * The pages describe a tile as a contiguous cube of tokens (podcast
 * transcript, the answer on what a tile is); this call makes each tile one
 * contiguous run of tau rows so that attention can stream it.
 *   x_raster: device, [B][heads][S][head_dim] raster order, read.
 *   x_tiled:  device, same size, written in tile-major order. No overlap.
 *   tile:     host int[3] (c_t, c_h, c_w), positive (see padding above).
 *   dtype:    sta_dtype; head_dim * element size must be a multiple of 16 bytes.
 */
int sta_reorder_tiles(const void* x_raster, void* x_tiled, int B, int heads, int head_dim,
                      int T, int H, int W, const int* tile, int dtype, void* stream);

/*
 * Inverse of sta_reorder_tiles: tile-major back to raster order (bit-exact),
 * so that the attention output returns to the token order of the model's
 * other layers (the pages' layout transformation: tokens are grouped into
 * contiguous tiles for the kernel and grouped back afterwards -- podcast
 * transcript, the answer on what a tile is; dianyo ICML2025 blog, Sparse
 * VideoGen, layout transformation). Padding rows of a tile-major input are
 * skipped. Same arguments, with the roles of input and output swapped.
 */
int sta_restore_order(const void* x_tiled, void* x_raster, int B, int heads, int head_dim,
                      int T, int H, int W, const int* tile, int dtype, void* stream);

/*
 * Enumerate, per head and query tile, the key tiles of its window: the
 * implicit block-sparse mask of STA (podcast transcript, the answers on the
 * producer warpgroups that hold the sparse mask and on the threadblock split).
 *   kv_list:  device int32 [heads][N_t][max_kv]; entries 0..count-1 hold the
 *             selected key tile indices in ascending order (raster order of
 *             tile coordinates), the rest are -1.
 *   kv_count: device int32 [heads][N_t]; omega_t * omega_h * omega_w.
 *   window:   host int[heads][3], tokens, each a multiple of the tile and at
 *             most the tile grid (n_a * c_a) on its axis.
 *   max_kv:   row length of kv_list; must be >= the largest count.
 * N_t = n_t * n_h * n_w.
 */
int sta_kv_tiles(int* kv_list, int* kv_count, int heads, int T, int H, int W, const int* tile,
                 const int* window, int max_kv, void* stream);

/*
 * The transposed relation: per head and key tile, the query tiles whose
 * window holds it, i.e. the query tiles that read the key tile and so
 * receive gradient from it. Needed by the backward pass, which is organised
 * by key tile; under the clamped window rule it differs from the key tiles'
 * own windows (a corner key tile is read by 2 x 2 x 2 query tiles at the
 * 30x48x80 / (6,8,8) / (18,24,24) geometry, a central one by 3 x 3 x 3 or
 * more). Per axis the query tiles form one contiguous interval.
 *   q_list:  device int32 [heads][N_t][max_q]; entries 0..count-1 hold the
 *            query tile indices in ascending order, the rest are -1.
 *   q_count: device int32 [heads][N_t].
 *   max_q:   row length of q_list; must be >= the longest list (else
 *            STA_ERR_INVALID_ARG, and sta_last_error() names the length).
 * Other arguments as sta_kv_tiles.
 */
int sta_q_tiles(int* q_list, int* q_count, int heads, int T, int H, int W, const int* tile,
                const int* window, int max_q, void* stream);

/*
 * Length of the longest tile list, for sizing the list buffers of
 * sta_kv_tiles (transposed = 0: the largest window, max_h prod_a omega_a) and
 * sta_q_tiles (transposed = 1: the most query tiles whose windows hold one
 * key tile). Host only; enqueues nothing. Arguments as sta_kv_tiles. Returns
 * the length (>= 1) or a negative sta_status.
 */
int sta_tile_list_len(int heads, int T, int H, int W, const int* tile, const int* window,
                      int transposed);

/*
 * Number of computed (query tile, key tile) pairs summed over heads, for one
 * batch entry: sum_h N_t * prod_a omega_a. This is the count of dense blocks
 * that STA computes instead of the N_t^2 blocks of full attention (atlas
 * summary, "Key results": the 91 % sparsity at w = (18,24,24) is
 * 1 - 27 / 300 of these pairs), and the effective TFLOP/s of the kernels are
 * counted from it. Host only; enqueues nothing.
 * Returns a negative sta_status on invalid arguments.
 */
long long sta_kv_pair_count(int heads, int T, int H, int W, const int* tile, const int* window);

/*
 * STA forward: for every batch entry b, head h and query tile i,
 *     O_i = softmax(scale * Q_i K_J^T) V_J,
 * with J the tokens of the key tiles in tile i's window (rule above) and the
 * softmax taken over those keys only. Softmax base e; only dense blocks are
 * computed (atlas.scime.ai summary, "Approach"; podcast transcript, the answer
 * on how blocks are computed). The window's key tiles are found inside the
 * kernel by the same integer rule as sta_kv_tiles.
 *   q, k, v: device [B][heads][S][head_dim] in TILE-MAJOR order, read.
 *   out:     device, same shape, tile-major, written. No overlap with inputs.
 *   tile:    host int[3]; window: host int[heads][3] (tokens), as above.
 *   scale:   finite, > 0 (1/sqrt(head_dim) is the usual choice).
 *   dtype:   STA_BF16 (head_dim 64 or 128) or STA_F32 (head_dim 64 or 128).
 * Accumulation is float32; for STA_BF16 the probabilities are rounded to
 * bfloat16 before they multiply V, and the output is rounded to bfloat16.
 */
int sta_forward(const void* q, const void* k, const void* v, void* out, int B, int heads,
                int head_dim, int T, int H, int W, const int* tile, const int* window,
                float scale, int dtype, void* stream);

/*
 * STA forward on raster-order tensors: the same result as sta_reorder_tiles of
 * q, k, v, then sta_forward, then sta_restore_order of the output, bit for bit,
 * in one kernel and without the intermediate tile-major copies. The grouping
 * of queries and keys into tiles (podcast transcript, the answer on what a tile
 * is) is folded into the kernel's addressing instead of a separate permutation.
 *   q, k, v: device [B][heads][S][head_dim] in RASTER order, read.
 *   out:     device, same shape, raster order, written. No overlap with inputs.
 * Other arguments and rules as sta_forward. Additionally each head's window run
 * omega_w * tau (keys that are consecutive in tile-major order) must be at most
 * 8192 keys, and one tile-row of frames, c_t * H * W tokens, must span less
 * than 2^31 bytes at 256 bytes a token (the kernels address a run's keys with
 * 32-bit offsets), else STA_ERR_UNSUPPORTED (reorder and call sta_forward
 * instead).
 */
int sta_forward_raster(const void* q, const void* k, const void* v, void* out, int B, int heads,
                       int head_dim, int T, int H, int W, const int* tile, const int* window,
                       float scale, int dtype, void* stream);

/*
 * STA forward that also writes, per query row, the log-sum-exp of its scores
 *     lse_i = log sum_j exp(scale * q_i . k_j)   over the row's window keys
 * (natural log, float32), which the backward pass needs to recompute the
 * probabilities. Output values are identical to sta_forward (order =
 * STA_TILE_MAJOR) or sta_forward_raster (order = STA_RASTER).
 *   lse:   device float [B][heads][S], 4-byte aligned, same token order as
 *          q; written. Must not overlap q, k, v or out.
 *   order: sta_order of q, k, v, out and lse.
 * Other arguments and rules as sta_forward / sta_forward_raster.
 */
int sta_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                    int heads, int head_dim, int T, int H, int W, const int* tile,
                    const int* window, float scale, int dtype, int order, void* stream);

/*
 * STA forward with fp8 queries and keys. The pages mention FP8 quantization
 * inside a sparse attention kernel (dianyo ICML2025 blog, Sparse VideoGen,
 * "Observation & Proposed Method"); here it applies to the score product:
 *     O_i = softmax(scale * (q_descale Q8_i) (k_descale K8_J)^T) V_J,
 * with Q8, K8 the values of the fp8 codes, window rule as sta_forward.
 *   q8, k8:  device uint8 [B][heads][S][128], OCP 8-bit floating point E4M3
 *            codes (bias 7, no infinities, 0x7F / 0xFF NaN, largest 448),
 *            read. The caller quantizes.
 *   v:       device bf16 [B][heads][S][128], read.
 *   out:     device bf16, same shape, written. No overlap with inputs.
 *   q_descale, k_descale: finite, > 0; per tensor. scale * q_descale *
 *            k_descale must be finite and > 0.
 *   order:   sta_order of q8, k8, v and out (tile-major or raster, with the
 *            rules of sta_forward and sta_forward_raster).
 * head_dim must be 128 (else STA_ERR_UNSUPPORTED). The fp8 products are exact
 * and summed in float32; probabilities and output are rounded to bfloat16 as
 * in sta_forward.
 */
int sta_forward_fp8(const void* q8, const void* k8, const void* v, void* out, int B, int heads,
                    int head_dim, int T, int H, int W, const int* tile, const int* window,
                    float scale, float q_descale, float k_descale, int order, void* stream);

/*
 * sta_forward_fp8 that also writes each query row's log-sum-exp of its scores
 * on the decoded values,
 *     lse_i = log sum_j exp(scale * (q_descale Q8_i) . (k_descale K8_j))
 * over the row's window keys (natural log, float32, summing the probabilities
 * as rounded to bfloat16 for the P V product, as sta_forward_lse does). The
 * decoded values times a power-of-two descale are bfloat16 values, so
 * training with fp8 scores (the fixed-window fine-tuning of the pages:
 * podcast transcript, the answer on fine-tuning; atlas.scime.ai summary,
 * "Approach") runs sta_backward on the decoded q and k with this lse.
 *   lse: device float [B][heads][S], 4-byte aligned, token order `order`;
 *        written. Must not overlap q8, k8, v or out.
 * Output values are identical to sta_forward_fp8's. Other arguments, rules
 * and errors as sta_forward_fp8.
 */
int sta_forward_fp8_lse(const void* q8, const void* k8, const void* v, void* out, float* lse, int B,
                        int heads, int head_dim, int T, int H, int W, const int* tile,
                        const int* window, float scale, float q_descale, float k_descale,
                        int order, void* stream);

/*
 * STA backward: gradients of sum(dout * O) with respect to q, k and v, for
 * training a model with a fixed STA window (the fine-tuning of the pages:
 * podcast transcript, the answer on fine-tuning; atlas.scime.ai summary,
 * "Approach"; dianyo ICML2025 blog, STA section). With P the window softmax
 * of the forward, recomputed as P_ij = exp(scale * q_i . k_j - lse_i):
 *     dV = P^T dO,  dS = P * (dO V^T - D),  D_i = dO_i . O_i,
 *     dQ = scale * dS K,  dK = scale * dS^T Q.
 *   q, k, v:    forward inputs; out: forward output O; dout: dO. Device,
 *               [B][heads][S][head_dim], token order `order`, read.
 *   lse:        device float [B][heads][S] from sta_forward_lse, read.
 *   dq, dk, dv: device, same shape and order as q, written (every element).
 *   delta:      device float [B][heads][S] workspace owned by the caller;
 *               overwritten with D. Must stay alive until the stream has
 *               passed the work.
 * Outputs and the workspace must not overlap any input or one another.
 * Accumulation is float32. For STA_BF16 the recomputed P and dS are rounded
 * to bfloat16 before they enter a matrix product, and the gradients are
 * rounded to bfloat16. Each gradient element is computed by one work item
 * (no atomics): results are deterministic. With order = STA_RASTER the
 * window runs and their transposes (the longest interval of query tiles
 * along w times tau) must be at most 8192 tokens and c_t * H * W tokens must
 * span less than 2^31 bytes at 256 bytes a token, else STA_ERR_UNSUPPORTED.
 * Other arguments and rules as sta_forward.
 */
int sta_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int heads,
                 int head_dim, int T, int H, int W, const int* tile, const int* window,
                 float scale, int dtype, int order, void* stream);

/*
 * sta_backward without the delta workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). D = rowsum(dO * O) goes to a static
 * 32 MiB device array that the library carries on every GPU it runs on
 * (until the process ends): B * heads * rows must be at most 8 Mi (8388608),
 * else STA_ERR_INVALID_ARG and nothing is enqueued. The call allocates
 * nothing. Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (other streams, other threads) race and must be serialised by
 * the caller. Arguments, outputs and results as sta_backward (bit-identical
 * gradients).
 */
int sta_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int heads, int head_dim, int T, int H, int W, const int* tile,
                         const int* window, float scale, int dtype, int order, void* stream);

/*
 * Window recall: for every batch entry b, head h and candidate window c,
 *     recall[b][h][c] = (1/S) sum_i sum_{j in W_c(i)} softmax_j(scale * q_i . k_j)
 * where the softmax runs over ALL S keys (full attention) and W_c(i) is the
 * key set of query i under candidate window c (the clamped tile window). It is
 * the share of full-attention probability a window keeps: the "attention
 * recall" the pages use to show that attention is local and to configure a
 * window per head by profiling (podcast transcript, the answers on attention
 * recall and on choosing the window per head; dianyo ICML2025 blog, STA
 * section, recall of local windows across prompts).
 * Computed as the mean of exp(lse_c(i) - lse_full(i)) from the row
 * log-sum-exps (the attention kernels in a log-sum-exp-only mode: no V, no
 * output; with bf16 inputs this mode sums the probabilities in float32
 * without rounding them to bfloat16, as nothing multiplies them), then a
 * deterministic double-precision reduction per (b, h). With bf16 (or fp8)
 * inputs, whole 64-key chunks per tile and no padding, one pass over all
 * keys (the whole volume as the window) per group of up to 8 candidates also
 * sums each candidate window's share, since every chunk lies in one key
 * tile; else a full-attention pass and one pass per candidate.
 *   q, k:        device [B][heads][S][head_dim], token order `order`, read.
 *   recall:      device float [B][heads][n_candidates], written.
 *   workspace:   device float [n_candidates + 1][B][heads][S], caller-owned;
 *                written with the row log-sum-exps over all keys (slot 0)
 *                and over each candidate's window (slot c + 1), in the
 *                token order of q.
 *   candidates:  host int[n_candidates][3], token windows, each valid for
 *                the volume and tile (same rule as `window`); applied to
 *                every head.
 * Dtype, head_dim, scale and the raster run limit as sta_forward_lse. No
 * buffer may overlap another.
 */
int sta_window_recall(const void* q, const void* k, float* recall, float* workspace, int B,
                      int heads, int head_dim, int T, int H, int W, const int* tile,
                      const int* candidates, int n_candidates, float scale, int dtype, int order,
                      void* stream);

/*
 * sta_window_recall on fp8 queries and keys: the recall of each candidate
 * window for the scores of sta_forward_fp8,
 *     scale * (q_descale Q8_i) . (k_descale K8_j),
 * so that windows are ranked on the same scores the fp8 forward computes
 * (recall and the per-head window choice: podcast transcript, the answers on
 * attention recall and on choosing the window per head; FP8 inside the sparse
 * attention kernel: dianyo ICML2025 blog, Sparse VideoGen, "Observation &
 * Proposed Method"). Both log-sum-exp passes sum the probabilities in
 * float32 without rounding them.
 *   q8, k8: device uint8 [B][heads][S][128], E4M3 codes as in
 *           sta_forward_fp8, token order `order`, read.
 *   q_descale, k_descale: finite, > 0.
 * head_dim must be 128 (else STA_ERR_UNSUPPORTED). Other arguments, buffers,
 * rules and errors as sta_window_recall.
 */
int sta_window_recall_fp8(const void* q8, const void* k8, float* recall, float* workspace, int B,
                          int heads, int head_dim, int T, int H, int W, const int* tile,
                          const int* candidates, int n_candidates, float scale, float q_descale,
                          float k_descale, int order, void* stream);

/*
 * Full softmax attention over all S keys (the computation STA replaces, used
 * as the speed-up denominator: atlas.scime.ai summary, "Key results").
 *   q, k, v, out: device [B][heads][S][head_dim], any common token order.
 * Same dtype, head_dim and scale rules as sta_forward; S >= 1, any length.
 */
int sta_full_attention(const void* q, const void* k, const void* v, void* out, int B, int heads,
                       int head_dim, int S, float scale, int dtype, void* stream);

/*
 * Message for the last non-OK status on this thread ("" if none). The pages
 * describe no interface; this is the error channel of the C boundary through
 * which the attention of the pages' video models is replaced (podcast
 * transcript, the opening answers on swapping full 3D attention for STA).
 */
const char* sta_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* STA_H_ */
