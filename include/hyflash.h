/*
 * libhyflash — the hot path of one HyFlash drafter layer on AMD MI355X (gfx950).
 *
 * HyFlash ("HyFlash: A Prefix-Memory Prior for On-Device Speculative Decoding")
 * drafts a block of seven future positions plus an anchor slot in one pass.  Each
 * drafter layer has two branches (HyFlash explainer, "That is HyFlash"):
 *   - a local-attention branch over the most recent committed target features and
 *     the block's own rows, in both directions;
 *   - a recurrent memory (Mamba-2) holding the committed history in a fixed-size
 *     state H, read while drafting and written only after verification, by the
 *     newly committed features alone (explainer FAQ, "Why does the memory update
 *     only from committed features?").
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns all memory:
 *     weights, the state pool, inputs, outputs and the workspace.  The library never
 *     allocates or frees device memory and keeps no mutable global state (one exception:
 *     hyf_draft_block_noalloc's per-GPU scratch array, see there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls only
 *     enqueue work on it and return without synchronizing.
 *   - Every call returns an hyf_status.  All conditions that can be checked on the
 *     host are checked before the first launch, so a call that returns an error other
 *     than HYF_EHIP has not touched device memory.  HYF_EHIP means a launch failed;
 *     the states named in that call are then undefined and must be reset.
 *   - Calls on different streams are safe when they name disjoint state slots and
 *     disjoint workspaces.
 *   - Storage dtype (cfg.dtype) applies to weights, features, block rows, ring K/V and
 *     outputs; the recurrent state H is always fp32 (explainer, "Where it earns its
 *     keep": the recurrent state is FP32).
 */
#ifndef HYFLASH_H
#define HYFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYF_ABI_VERSION 2
/* Requests per call (state slots touched by one commit or draft call). */
#define HYF_MAX_REQUESTS 128
/* Rows of the draft block: anchor + seven draft positions (explainer, "Jargon"). */
#define HYF_BLOCK 8
/* Tokens per block of the time-blocked layout hyf_ssd_scan reads (see there). */
#define HYF_TBLK 128

typedef enum {
  HYF_OK = 0,
  HYF_EINVAL = 1,       /* null pointer, misaligned pointer, bad count or offsets   */
  HYF_ESHAPE = 2,       /* unsupported or inconsistent shape                         */
  HYF_ECAPACITY = 3,    /* too many requests or rows, slot outside the pool          */
  HYF_EDTYPE = 4,       /* unknown dtype                                             */
  HYF_EWORKSPACE = 5,   /* ws_bytes smaller than the size the matching query returns */
  HYF_EUNSUPPORTED = 6, /* a mode the library does not implement                     */
  HYF_EHIP = 7          /* a HIP launch failed                                       */
} hyf_status;

typedef enum { HYF_F32 = 0, HYF_BF16 = 1 } hyf_dtype;
/* The recurrent memory: Mamba-2 over the whole committed history; the gated delta rule in its place
 * (the paper's memory ablation, Gated DeltaNet-2); or Mamba-2 over the last W committed rows only
 * (the paper's history ablation, "SSM: last 512": HyFlash paper page, Figures & tables, the
 * ablation table; explainer, "That is HyFlash", the paragraph on the ablations). */
typedef enum { HYF_MEM_MAMBA2 = 0, HYF_MEM_GDN = 1, HYF_MEM_LASTW = 2 } hyf_memory;
/* Weights of the layer's two projections: in the storage dtype, or 4-bit codes with fp32 scales
 * (HyFlash paper page, Figures & tables: the BF16 vs INT4 table; explainer, "Where it earns its
 * keep": the drafter's weights quantized to 4 bits keep the bf16 drafter's acceptance). */
typedef enum { HYF_WEIGHTS_DENSE = 0, HYF_WEIGHTS_W4 = 1 } hyf_weight_format;

/* Layer shape.  48 bytes, all int32. */
typedef struct {
  int32_t d_model;    /* d                                                             */
  int32_t n_heads;    /* nh; attention heads = memory heads; nh*head_dim is the q/k/v width */
  int32_t head_dim;   /* P: multiple of 16, at most 256                                 */
  int32_t d_state;    /* N: multiple of 16, at most 256                                 */
  int32_t n_groups;   /* G: B and C are shared by nh/G heads each; must divide nh       */
  int32_t window;     /* W: ring capacity in committed rows (1..8192)                   */
  int32_t block;      /* must be HYF_BLOCK                                             */
  int32_t chunk;      /* SSD chunk length L: a power of two, 16..1024                   */
  int32_t dtype;      /* hyf_dtype                                                      */
  int32_t memory;     /* hyf_memory (HYF_MEM_GDN: see hyf_weights; HYF_MEM_LASTW: see the
                         state layout and hyf_memory_commit)                              */
  int32_t cross_slot; /* 1: block rows attend to each other; 0: each only to itself     */
  int32_t weights;    /* hyf_weight_format; HYF_WEIGHTS_W4 needs HYF_BF16 and d_model and
                         nh*head_dim multiples of 128 (HYF_EUNSUPPORTED otherwise)          */
} hyf_config;

/* Layer weights, nn.Linear layout ([out_features][in_features], row-major).
 * w_in rows come in groups, in this order:
 *   q [nh*P] | C [G*N] | k [nh*P] | v [nh*P] | B [G*N] | dt [nh]      (n_in rows in all)
 * The value projection v is also the memory's input x.  a_log, dt_bias and d_skip are
 * fp32 per head: A = -exp(a_log), dt = softplus(raw + dt_bias), D = d_skip.
 *
 * memory = HYF_MEM_GDN, the gated delta-rule memory the HyFlash paper's memory ablation swaps in
 * for Mamba-2 (Gated DeltaNet-2): w_in ends | B [G*N] | alpha [nh] | beta [nh], so n_in has nh
 * more rows; per head and committed row, with k = B / sqrt(|B|^2 + 1e-6),
 *   alpha = sigmoid(raw_alpha + dt_bias[h]),  beta = sigmoid(raw_beta + a_log[h]),
 *   H <- alpha H (I - beta k k^T) + beta v k^T,
 * and the readout uses C_q / sqrt(|C_q|^2 + 1e-6).  (dt_bias and a_log carry the two gate biases.)
 * Per-token outputs (y_opt) and hyf_ssd_scan are Mamba-2 only (HYF_EUNSUPPORTED); a commit of more
 * than 16 rows per request needs d_state <= 192, or d_state 224 in bf16 (HYF_EUNSUPPORTED otherwise). */
typedef struct {
  const void* w_in;     /* [n_in][d_model], storage dtype, 16-byte aligned (dense weights)   */
  const void* w_out;    /* [d_model][nh*P], storage dtype, 16-byte aligned (dense weights)   */
  const float* a_log;   /* [nh] */
  const float* dt_bias; /* [nh] */
  const float* d_skip;  /* [nh] */
  /* 4-bit weights (cfg->weights = HYF_WEIGHTS_W4; w_in and w_out are then not read): the same
   * matrices as codes 0..15 standing for (code - 8) * scale, two per byte along the input
   * dimension (the lower index in the low nibble), one fp32 scale per 128 consecutive inputs of a
   * row, as hyf_linear_w4 takes them.  Codes 16-byte aligned, scales 4-byte aligned. */
  const uint8_t* w_in_q;  /* [n_in][d_model / 2]        */
  const float* w_in_s;    /* [n_in][d_model / 128]      */
  const uint8_t* w_out_q; /* [d_model][nh*P / 2]        */
  const float* w_out_s;   /* [d_model][nh*P / 128]      */
} hyf_weights;

/* Byte offsets inside one request's state blob (each section 256-byte aligned):
 *   header: int64 committed count at offset 0 (the ring head is count mod W), rest 0
 *   H:      fp32 [nh][P][N]
 *   K, V:   storage dtype [nh][W][P]; committed row c of the request sits in slot c mod W
 *   B ring: storage dtype [W][G*N], the B row of the row in each slot      (HYF_MEM_LASTW only)
 *   step ring: fp32 [nh][W], the raw step (before dt_bias) of each slot     (HYF_MEM_LASTW only)
 * b_off and dt_off are 0 when the memory keeps no B and step rings. */
typedef struct {
  uint64_t count_off, h_off, k_off, v_off, total, b_off, dt_off;
} hyf_state_layout;

int hyf_abi_version(void);
const char* hyf_status_str(int status);

/* Host only.  HYF_OK if cfg describes a shape the library runs. */
int hyf_config_check(const hyf_config* cfg);

/* Host only.  Size of the input projection's output (n_in above); 0 on a bad cfg. */
int64_t hyf_n_in(const hyf_config* cfg);

/* Host only.  Fills *out; one request's state for one layer. */
int hyf_state_layout_get(const hyf_config* cfg, hyf_state_layout* out);
/* Host only.  Bytes of one state blob (= layout.total, a multiple of 256); 0 on a bad cfg.
 * A state pool is pool_slots blobs back to back. */
size_t hyf_state_bytes(const hyf_config* cfg);

/* Host only.  Workspace bytes that hyf_memory_commit and hyf_draft_block need for up to
 * max_requests requests and up to max_rows committed rows in one call (summed over the
 * requests); with_y != 0 sizes it for hyf_memory_commit with per-token outputs (y_opt), which
 * keeps one P x N state per 128 committed rows.  0 on bad arguments. */
size_t hyf_workspace_bytes(const hyf_config* cfg, int32_t max_requests, int64_t max_rows, int32_t with_y);

/* Empties the named states: count = 0, H = 0, ring zeroed.
 * slots (host, nullable): pool index of each request; NULL means 0..n_req-1. */
int hyf_state_reset(const hyf_config* cfg, void* state_pool, int32_t pool_slots,
                    const int32_t* slots, int32_t n_req, void* stream);

/* With memory = HYF_MEM_LASTW a commit appends k, v, B and the raw step of its rows to the rings,
 * then rebuilds H from zero as the Mamba-2 scan of the last min(count, W) committed rows in commit
 * order (from the stored, rounded x = v, B and steps); drafting reads that H like any other.  A
 * draft call with commit rows then runs the commit and the draft one after the other (no fused
 * projection pass).  Per-token outputs (y_opt) are HYF_EUNSUPPORTED. */

/* With 4-bit weights a round's projections (hyf_draft_block, and hyf_memory_commit of at most 16
 * rows per request) compute with the codes exactly (as hyf_linear_w4); a longer commit first
 * expands the codes of the w_in rows it uses to bf16 values (code - 8) * scale in the workspace
 * and runs the bf16 prefill GEMM on them. */

/* Commit: the only writer of committed state (explainer, "That is HyFlash": after
 * verification only the newly committed features update the memory).
 * Request i folds rows feats[cu_rows[i] .. cu_rows[i+1]) — its newly committed target
 * features, [rows][d_model] in storage dtype — into its state, in order:
 *   k, v, B, dt_raw from w_in; H <- exp(dt*A) H + dt * (v outer B) token by token
 *   (computed as a chunked scan); the last min(rows, W) (k, v) pairs enter the ring at
 *   slots (count + j) mod W; count += rows.
 * Any row count works (a prefill of a whole prefix, or the 1-8 rows of a round).
 * cu_rows (host): int64 [n_req + 1], cu_rows[0] = 0, non-decreasing.  Empty requests
 * are left bit-identical.
 * With memory = HYF_MEM_GDN the fold is the gated delta rule of hyf_weights, the same result as
 * row by row (computed, for more than 16 rows, in chunks of 64 tokens: per-chunk triangular
 * solves, then one state update per chunk; the workspace then holds (N + P + 1) * 64 + 4 floats
 * per chunk and head, which hyf_workspace_bytes includes); y_opt is HYF_EUNSUPPORTED.
 * y_opt (nullable, 16-byte aligned): [cu_rows[n_req]][nh][P] storage dtype, per-token memory
 * outputs y_t = H_t . C_t + D * v_t (H_t after token t, C_t from w_in); HYF_EUNSUPPORTED when
 * the staged 128-token block does not fit one workgroup's LDS: x, B and C for fp32 (P + 2N >= 320)
 * and for bf16 heads of more than 128 dimensions (P + 2N >= 640); B and C alone for other bf16
 * heads, which always fit.
 * ws: at least hyf_workspace_bytes(cfg, n_req, cu_rows[n_req], y_opt != NULL) bytes, 256-byte
 * aligned. */
int hyf_memory_commit(const hyf_config* cfg, const hyf_weights* w, void* state_pool,
                      int32_t pool_slots, const int32_t* slots, int32_t n_req, const void* feats,
                      const int64_t* cu_commit, void* y_opt, void* ws, size_t ws_bytes,
                      void* stream);

/* One draft step for n_req requests (paper Abstract; explainer "That is HyFlash").
 * If commit_feats is not NULL, the call first performs exactly hyf_memory_commit on those
 * rows (cu_commit (host) as cu_rows above, at most `block` rows per request), sharing one
 * pass over w_in with the block rows.  Then, per request and head, with block rows
 * block_in [n_req][block][d_model]:
 *   q, k, v, C_q from w_in;
 *   attn = softmax(q . keys / sqrt(P)) . values, keys = the last min(count, W) committed
 *          rows in the ring plus all block rows (no causal mask; cross_slot = 0 hides the
 *          other block rows);
 *   mem  = H . C_q + D * v   (H is read, never written);
 *   block_out [n_req][block][d_model] = concat_heads(attn + mem) . w_out^T.
 * Drafting never writes the state: with commit_feats == NULL the state pool is left bit-
 * identical.  ws: at least hyf_workspace_bytes(cfg, n_req, cu_commit[n_req], 0) bytes. */
int hyf_draft_block(const hyf_config* cfg, const hyf_weights* w, void* state_pool,
                    int32_t pool_slots, const int32_t* slots, int32_t n_req,
                    const void* commit_feats, const int64_t* cu_commit, const void* block_in,
                    void* block_out, void* ws, size_t ws_bytes, void* stream);

/* Size of the device array hyf_draft_block_noalloc uses in place of a workspace (16 MiB). */
#define HYF_NOALLOC_SCRATCH_BYTES (16u << 20)

/* hyf_draft_block without a workspace argument, for callers that cannot allocate device memory
 * (code that runs under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, checks, kernels and results as hyf_draft_block (bit for bit); the workspace is a
 * device array of HYF_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the first
 * call on that GPU (with it current) until the process ends.  The call allocates and frees
 * nothing.  Calls whose draft workspace would exceed the array (it grows with n_req and the
 * commit rows; one request of a layer up to d_model 5120 with 40 heads of 128 fits, at the
 * Qwen3-4B-shaped layer about ten) return HYF_ECAPACITY before any device work.  Every call on one GPU shares that GPU's array, so calls that overlap
 * on one GPU (other streams, other threads) race: the caller orders them.  The stream must belong
 * to the current device. */
int hyf_draft_block_noalloc(const hyf_config* cfg, const hyf_weights* w, void* state_pool,
                            int32_t pool_slots, const int32_t* slots, int32_t n_req,
                            const void* commit_feats, const int64_t* cu_commit,
                            const void* block_in, void* block_out, void* stream);

/* hyf_draft_block with the round's accepted-row counts on the device, for a serving loop whose
 * verification step leaves them in GPU memory (explainer, "That is HyFlash": the accepted rows are
 * committed before the next block is drafted): no host array depends on the counts, so one call
 * has fixed launch shapes and can be captured in a graph once and replayed every round.
 * commit_feats: [n_req][HYF_BLOCK][d_model] storage dtype, request i's committed row j at row
 * i*HYF_BLOCK + j (rows past its count are projected and ignored; they may hold anything);
 * commit_rows: device int32 [n_req], request i commits commit_rows[i] rows (values outside
 * 0..HYF_BLOCK are clamped), read by the kernels when they run; both NULL for a pure draft.
 * Results equal hyf_draft_block's for the same rows.  ws: at least
 * hyf_workspace_bytes(cfg, n_req, HYF_BLOCK * n_req, 0) bytes. */
int hyf_draft_block_dev(const hyf_config* cfg, const hyf_weights* w, void* state_pool,
                        int32_t pool_slots, const int32_t* slots, int32_t n_req,
                        const void* commit_feats, const int32_t* commit_rows,
                        const void* block_in, void* block_out, void* ws, size_t ws_bytes,
                        void* stream);

/* The projection building block of the layer (explainer, "That is HyFlash": each layer
 * projects committed features and block rows; the draft step ends in an output projection):
 *   out[m][f] = sum_k X[m][k] * W[f][k]      m < M, f < Nout
 * X [M][K] and W [Nout][K] (nn.Linear layout) in the storage dtype, 16-byte aligned, K a
 * multiple of 8; out [M][Nout] is fp32 when out_f32 != 0, else the storage dtype.  It runs the
 * same kernels, with the same launch shapes, as hyf_draft_block and hyf_memory_commit do for
 * the same M and K (a weight-streaming kernel up to 64 rows, a tiled MFMA GEMM above). */
int hyf_linear(const hyf_config* cfg, const void* X, int64_t M, int32_t K, const void* W,
               int32_t Nout, void* out, int32_t out_f32, void* stream);

/* Weight-only 4-bit projection (paper page, Figures & tables: a 4-bit drafter keeps the bf16
 * drafter's acceptance; explainer, "Where it earns its keep": the drafter's weights in 4 bits):
 *   out[m][f] = sum_k X[m][k] * (code(f, k) - 8) * scales[f][k / 128]      m < M, f < Nout
 * X [M][K] bf16 (cfg->dtype must be HYF_BF16, else HYF_EUNSUPPORTED), 16-byte aligned.
 * Wq [Nout][K/2] bytes, 16-byte aligned: codes 0..15, two per byte along k, the lower k in the
 * low nibble.  scales [Nout][K/128] fp32, 4-byte aligned.  K a multiple of 128, 1 <= Nout <=
 * 2^24, 0 <= M <= 64 * 65535 (HYF_ESHAPE otherwise).  out [M][Nout] is fp32 when out_f32 != 0,
 * else bf16.  All device pointers, owned by the caller; M = 0 is a no-op.  The weights are
 * streamed once per 64 rows of X, so the call suits round-sized M (up to 64 rows). */
int hyf_linear_w4(const hyf_config* cfg, const void* X, int64_t M, int32_t K, const void* Wq,
                  const float* scales, int32_t Nout, void* out, int32_t out_f32, void* stream);

/* The full drafter block around the two-branch layer.  The pages fix the layer (explainer, "That
 * is HyFlash": every drafter layer holds a local-attention branch and the recurrent memory) and a
 * drafter backbone of a few milliseconds ("Where it earns its keep"), not the blocks around it;
 * the plainest pre-norm residual block is:
 *   h   = x + Layer(RMSNorm(x) * norm1)
 *   out = h + (silu(z . w_gate^T) * (z . w_up^T)) . w_down^T,   z = RMSNorm(h) * norm2,
 *   RMSNorm(x) = x / sqrt(mean over d_model of x^2 + eps),
 * and the memory commits the layer's own input, RMSNorm(feats) * norm1.  Layer is the
 * hyf_draft_block / hyf_memory_commit layer of hyf_weights.
 * norm1, norm2 [d_model] fp32; w_gate_up [2 d_ff][d_model] storage dtype, the gate rows first
 * (rows 0 .. d_ff - 1), then the up rows; w_down [d_model][d_ff] storage dtype; all 16-byte
 * aligned device pointers owned by the caller.  d_ff >= 16, a multiple of 16 (HYF_ESHAPE
 * otherwise); eps >= 0.  4-bit layer weights are allowed; the block's own weights are dense. */
typedef struct {
  const float* norm1;
  const float* norm2;
  const void* w_gate_up;
  const void* w_down;
  int32_t d_ff;
  float eps;
} hyf_block_weights;

/* Host only.  Workspace bytes hyf_block_commit and hyf_block_draft need for up to max_requests
 * requests and max_rows committed rows per call (0 for invalid arguments). */
size_t hyf_block_workspace_bytes(const hyf_config* cfg, const hyf_block_weights* bw, int32_t max_requests,
                                 int64_t max_rows);

/* The block's commit: hyf_memory_commit of RMSNorm(feats) * norm1 (arguments as there, without
 * per-token outputs).  ws: at least hyf_block_workspace_bytes(cfg, bw, n_req, cu_rows[n_req]). */
int hyf_block_commit(const hyf_config* cfg, const hyf_weights* w, const hyf_block_weights* bw,
                     void* state_pool, int32_t pool_slots, const int32_t* slots, int32_t n_req,
                     const void* feats, const int64_t* cu_rows, void* ws, size_t ws_bytes, void* stream);

/* One draft step of the block: with commit_feats not NULL, exactly hyf_block_commit of those rows
 * first (at most `block` rows per request, as hyf_draft_block); then block_out
 * [n_req][block][d_model] (storage dtype) = out above for block_in [n_req][block][d_model].
 * Never writes the state when commit_feats is NULL.  block_out must not overlap block_in.
 * ws: at least hyf_block_workspace_bytes(cfg, bw, n_req, cu_commit[n_req]) bytes. */
int hyf_block_draft(const hyf_config* cfg, const hyf_weights* w, const hyf_block_weights* bw,
                    void* state_pool, int32_t pool_slots, const int32_t* slots, int32_t n_req,
                    const void* commit_feats, const int64_t* cu_commit, const void* block_in,
                    void* block_out, void* ws, size_t ws_bytes, void* stream);

/* Host only.  Workspace bytes hyf_ssd_scan needs for T tokens, with (with_y != 0) or without
 * per-token outputs. */
size_t hyf_ssd_scan_workspace_bytes(const hyf_config* cfg, int64_t T, int32_t with_y);

/* The memory's scan on pre-projected inputs, one request (explainer "Jargon": Mamba-2 folds
 * each input into a fixed-size state with an input-dependent step size and a learned decay).
 * For t = 0..T-1, per head h (g(h) = h / (nh/G)):
 *   dt = softplus(dt_raw(h,t) + dt_bias[h]);  H_h <- exp(dt * A_h) H_h + dt * x(h,t) outer B(g(h),t)
 *   y[t][h] = H_h . C(g(h),t) + d_skip[h] * x(h,t)              (only if y_opt)
 * Inputs are time-blocked: tokens come in blocks of HYF_TBLK; a tensor of F features holds
 * ceil(T / HYF_TBLK) blocks of F * HYF_TBLK elements, block b holding tokens b*HYF_TBLK .. +127.
 *   dt_raw F = nh    fp32, plain: feature f of token t at (t / HYF_TBLK) * F * HYF_TBLK +
 *                    f * HYF_TBLK + t % HYF_TBLK;
 *   x      F = nh*P  storage dtype, feature h*P + p, tiled;
 *   B, C   F = G*N   storage dtype, feature g*N + n, tiled (C_opt is required iff y_opt is given).
 * Tiled (the operand order of the 16x16 MFMAs that consume it): with VN = 16 / sizeof(element)
 * (8 bf16, 4 fp32), KT = 4*VN and NJ = HYF_TBLK / KT, feature f of token t sits in its block at
 *   (((f / 16) * NJ + (t % HYF_TBLK) / KT) * 64 + ((t % KT) / VN) * 16 + f % 16) * VN + t % VN,
 * i.e. each group of 16 features and run of KT tokens is one contiguous 1 KiB tile.
 * Entries of the last block past T are never read into the result (they may hold anything).
 * x, B and dt_raw 16-byte aligned.
 * H_inout [nh][P][N] fp32 holds the initial state on entry and the final state on exit.
 * y_opt [T][nh][P] storage dtype, 16-byte aligned (HYF_EUNSUPPORTED as for hyf_memory_commit).
 * ws: at least hyf_ssd_scan_workspace_bytes(cfg, T, y_opt != NULL) bytes.  T = 0 is a no-op. */
int hyf_ssd_scan(const hyf_config* cfg, const void* x, const void* B, const void* C_opt,
                 const float* dt_raw, const float* a_log, const float* dt_bias,
                 const float* d_skip, float* H_inout, void* y_opt, int64_t T, void* ws,
                 size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HYFLASH_H */
