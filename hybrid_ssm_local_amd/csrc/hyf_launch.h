// Host-side launchers of the libhyflash kernels (implemented in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hyf_device.h"

namespace hyf {

// Where a projection writes its output columns: columns < n_split go to out0 (fp32 when
// out0_f32, else the storage dtype) with row stride ld0; columns >= n_split go to out1 (fp32)
// at column (col - n_split) with row stride ld1.  With trans != 0 the output is written
// time-blocked instead (rows m are tokens, blocks of HYF_TBLK; ld0 and ld1 are block strides):
// out0 in the tiled layout of tile_off (storage dtype) or plain [f][HYF_TBLK] rows (fp32), out1
// in plain rows.  If zero is set, the launch also clears zero[0 .. n_zero) (the counters of the
// kernel that consumes this output).
struct Epi {
  void* out0;
  int64_t ld0;
  int32_t out0_f32;
  int32_t n_split;
  float* out1;
  int64_t ld1;
  int32_t trans;
  int32_t* zero;
  int32_t n_zero;
};

// Rows of the projection input: rows m < M1 come from X1 (row stride K), the rest from X2.
struct RowSrc {
  const void* X1;
  const void* X2;
  int64_t M1;
};

// Store of output element (row m, feature f) through an epilogue description.
template <typename T>
__device__ __forceinline__ void epi_store(const Epi& e, int64_t m, int f, float v) {
  if (e.trans) {
    const int64_t blk = m / HYF_TBLK, off = m % HYF_TBLK;
    if (f < e.n_split) {
      // out0: the tiled layout of the storage dtype (or plain [f][HYF_TBLK] for fp32 output)
      if (e.out0_f32)
        static_cast<float*>(e.out0)[blk * e.ld0 + (int64_t)f * HYF_TBLK + off] = v;
      else
        static_cast<T*>(e.out0)[blk * e.ld0 + tile_off<T>(f, (int)off)] = from_f32<T>(v);
    } else {
      e.out1[blk * e.ld1 + (int64_t)(f - e.n_split) * HYF_TBLK + off] = v;
    }
    return;
  }
  if (f < e.n_split) {
    if (e.out0_f32)
      static_cast<float*>(e.out0)[m * e.ld0 + f] = v;
    else
      static_cast<T*>(e.out0)[m * e.ld0 + f] = from_f32<T>(v);
  } else {
    e.out1[m * e.ld1 + (f - e.n_split)] = v;
  }
}

__device__ __forceinline__ const void* row_ptr(const RowSrc& xs, int64_t m, int K, int esz) {
  if (m < xs.M1) return static_cast<const char*>(xs.X1) + m * (int64_t)K * esz;
  return static_cast<const char*>(xs.X2) + (m - xs.M1) * (int64_t)K * esz;
}

// out[m][f] = sum_k X[m][k] * W[f][k]   for m < M, f < Nout (W is [Nout][K], row-major).
// Picks the weight-streaming kernel (small M) or the tiled MFMA GEMM (large M).
hipError_t launch_linear(int dtype, RowSrc x, int64_t M, int K, const void* W, int Nout,
                         const Epi& epi, hipStream_t s);
// Weight-only 4-bit projection (hyf_w4.hip); K a multiple of 128.
hipError_t launch_linear_w4(const bf16* X, int64_t M, int K, const uint8_t* Wq, const float* S, int Nout,
                            void* out, bool out_f32, hipStream_t s);
// The same with rows from a RowSrc and the output through an epilogue description (not time-blocked).
hipError_t launch_linear_w4_epi(const RowSrc& x, int64_t M, int K, const uint8_t* Wq, const float* S, int Nout,
                                const Epi& epi, hipStream_t s);
// bf16 values (code - 8) * scale of `rows` rows of 4-bit weights with K inputs each: out [rows][K].
hipError_t launch_w4_dequant(const uint8_t* Wq, const float* S, int rows, int K, bf16* out, hipStream_t s);
// The tiled bf16 GEMM (hyf_gemm.hip); K must be a multiple of 64.
hipError_t launch_gemm256(RowSrc x, int M, int K, const bf16* W, int Nout, const Epi& epi, hipStream_t s);

// The full drafter block's row kernels (hyf_block.hip); rows of d (or F) elements, contiguous.
// y = RMSNorm(x) * g (storage dtype in and out).
hipError_t launch_rmsnorm(int dtype, const void* x, int64_t rows, int d, const float* g, float eps, void* y,
                          hipStream_t s);
// h = x + o (fp32) and z = RMSNorm(h) * g (storage dtype).
hipError_t launch_resid_norm(int dtype, const void* x, const void* o, int64_t rows, int d, const float* g, float eps,
                             float* h, void* z, hipStream_t s);
// a[m][j] = silu(gu[m][j]) * gu[m][F + j] (gu fp32 [rows][2F], a storage dtype [rows][F]).
hipError_t launch_swiglu(int dtype, const float* gu, int64_t rows, int F, void* a, hipStream_t s);
// out = h + y over n elements (fp32 in, storage dtype out).
hipError_t launch_add_out(int dtype, const float* h, const float* y, int64_t n, void* out, hipStream_t s);

// Rows of a grouped product: one GEMM launch over the rows of several requests.  Product row m
// belongs to the group g with m0[g] <= m < m0[g + 1]; its local index is l = m - m0[g], and only
// l < cnt[g] is a row of the group (rows past cnt[g], up to the next group, are padding: computed
// from the group's last row and never stored).  Row l reads input row src0[g] + l of X and, with a
// time-blocked epilogue (epi.trans), writes token l of a sequence whose first block is blk0[g]
// (in blocks of the epilogue's strides); a row-major epilogue writes product row m.  A time-blocked
// product needs every m0[g] to be a multiple of 8.  Groups may be empty.
struct RowGroups {
  int32_t n;
  int32_t m0[HYF_MAX_REQUESTS + 1];
  int32_t cnt[HYF_MAX_REQUESTS];
  int32_t src0[HYF_MAX_REQUESTS];
  int32_t blk0[HYF_MAX_REQUESTS];
};
// out = X[rows of g] . W^T over all groups in one launch (bf16, K a multiple of 64, rows from X with
// row stride K).
hipError_t launch_gemm_grouped(const bf16* X, const RowGroups& g, int K, const bf16* W, int Nout, const Epi& epi,
                               hipStream_t s);

// Memory scan over segments (see hyf_scan.hip).  Inputs are time-blocked: token t of request i
// sits in block blk0[i] + t / HYF_TBLK (block stride *blk); x, B and C are tiled inside a block
// (tile_off), dt is plain ([feature][HYF_TBLK]).
struct ScanArgs {
  const void* x;      // x, feature h*P + p
  const void* B;      // B, feature g*N + n
  const float* dt;    // raw step (before bias), feature h
  int64_t xblk, bblk, dblk;  // block strides (elements) of x, B and dt
  const float* a_log;
  const float* dt_bias;
  char* state_pool;   // H of request i at state_pool + slot*st_bytes + st_h (if h_direct == null)
  float* h_direct;    // single-request H (hyf_ssd_scan); overrides the pool when non-null
  float* part;        // [total_segs][nh][P][N] partial states
  float* lam;         // [total_segs][nh] segment log-decays
  int32_t seg_tokens; // tokens per segment (a multiple of HYF_TBLK; the last one may be short)
  int32_t total_segs;
  // per-token outputs (y-mode: segments of HYF_TBLK tokens; part then holds each segment's
  // starting state): y [rows][nh][P] storage dtype, row = request row0 + token
  int32_t y_mode;
  const void* C;      // C, feature g*N + n, tiled like B
  int64_t cblk;
  void* y;
  const float* d_skip;
};
// Longest segment (tokens) one scan workgroup takes: its per-token weights live in LDS.
int64_t scan_max_seg_tokens(const Shape& sh, int esz);
// Whether the y-mode kernel fits this shape (its segment's x, B, C live in LDS).
bool scan_y_supported(const Shape& sh, int esz);
// Scan workgroups per segment: heads x P-blocks x N-blocks.
int64_t scan_items_per_seg(const Shape& sh);
hipError_t launch_ssd_state(int dtype, const Shape& sh, const ScanArgs& a, const ReqTable& rt,
                            int32_t max_segs_per_req, hipStream_t s);

// Round kernel (see hyf_round.hip).
// Division of small non-negative indices by a divisor d >= 1 as one multiply-high: with
// m = ceil(2^32 / d), floor(i / d) = mulhi(i, m) exactly whenever i d < 2^32 (0 <= m d - 2^32 < d);
// d = 1 wraps m to 0 and is taken apart.  Built on the host, so kernels divide without a sequence.
struct Div {
  uint32_t m;
  int32_t d;
  Div() = default;
  __host__ __device__ explicit Div(int d_) : m(0xFFFFFFFFu / (uint32_t)d_ + 1u), d(d_) {}
  __device__ int q(int i) const { return m ? (int)__umulhi((uint32_t)i, m) : i; }
  __device__ int r(int i) const { return i - q(i) * d; }
};

struct RoundArgs {
  const float* proj;   // [rows][ld] fp32: commit rows first (row0 table), then block rows
  int64_t ld;          // row stride of proj (n_in rounded up to a multiple of 4)
  int64_t blk_row0;    // first block row in proj
  char* state_pool;
  const float* a_log;
  const float* dt_bias;
  const float* d_skip;
  float* mem;          // [n_req][8][nh][P]
  float* att_part;     // [n_req][nh][n_split][8][P]
  float* att_ml;       // [n_req][nh][n_split][8][2]
  void* o_in;          // [n_req*8][dq] storage dtype
  int32_t* counters;   // [n_req*nh + n_req], zero on entry
  int32_t n_tiles;     // commit / readout tiles per (request, head)
  int32_t n_split;     // attention splits per (request, head), the last one holds the block keys
  int32_t do_commit;   // commit rows present
  int32_t do_draft;    // block rows present
  int32_t tile_rows;   // rows of H per commit / readout tile
  int32_t ks;          // ring slots per attention split
  // nullable: committed rows of request r read from device memory (clamped to 0..HYF_BLOCK); its
  // commit rows then sit at proj rows HYF_BLOCK r .. (a padded layout) instead of the table's row0
  const int32_t* dev_rows;
  // set by launch_round: n_tiles + n_split, nh, P / 4, P, N / 4, tile_rows
  Div d_per, d_nh, d_p4, d_p, d_tpr, d_tr;
};
// Fills n_tiles, tile_rows, ks and n_split of a round over n_req requests (esz: storage bytes).
void round_layout(const Shape& sh, int n_req, int esz, RoundArgs* a);
// The most attention splits any layout uses (the workspace is sized for it).
int round_max_splits(const Shape& sh);

// Gated delta-rule commit of whole prefixes (sh.gdn): x and B tiled as for the Mamba-2 scan, the raw
// gates time-blocked in a.dt (alpha at feature h, beta at nh + h, block stride a.dblk); gate biases
// in a.dt_bias (alpha) and a.a_log (beta); updates the state pool's H in place.
bool gdn_supported(const Shape& sh);
// The chunked form (chunks of 64 tokens: per-chunk solves, then a chain over chunks) runs when the
// shape allows it; it then needs rt.seg0 to hold each request's first chunk and a.part to hold
// gdn_chunk_record_floats(sh) floats per (chunk, head).
bool gdn_chunked_supported(const Shape& sh, int esz);
int64_t gdn_chunk_record_floats(const Shape& sh);
constexpr int GDN_CHUNK = 64;
hipError_t launch_gdn_commit(int dtype, const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s);
hipError_t launch_round(int dtype, const Shape& sh, const RoundArgs& a, const ReqTable& rt, hipStream_t s);

// Prefill ring append: the last m_i = min(n_i, W) rows of request i go to slots
// (count + n_i - m_i + j) mod W.  k: token-major [sum m_i][ld_k] (the requests' last rows back to
// back); v: time-blocked with block stride ld_v (feature h*P + p, token n_i - m_i + j); with the
// last-W memory also B (feature dq + g*N + n of the same buffer) and the raw step (dtT, plain,
// block stride ld_dt) into the B and step rings.
hipError_t launch_ring_append(int dtype, const Shape& sh, char* pool, const ReqTable& rt,
                              const void* k, int64_t ld_k, const void* vT, int64_t ld_v,
                              const float* dtT, int64_t ld_dt, hipStream_t s);
// The last-W memory's rescan input: request i's window (rt.slot[i], its count already advanced) as
// W rows in commit order, the first W - min(count, W) of them padding (x = 0, B = 0, step 0),
// written time-blocked like the prefill's (x | B tiled with block stride ld_vb starting at block
// rt.blk0[i]; raw steps plain with block stride ld_dt); H of each request zeroed.
hipError_t launch_lastw_gather(int dtype, const Shape& sh, char* pool, const ReqTable& rt, void* vb, int64_t ld_vb,
                               float* dtT, int64_t ld_dt, hipStream_t s);
// count += rows committed, per request (the last launch of a commit).
hipError_t launch_bump_counts(char* pool, const Shape& sh, const ReqTable& rt, hipStream_t s);
// Zero fill (a kernel, not a memset, so graph replays stay correct).
hipError_t launch_zero(void* p, uint64_t bytes, hipStream_t s);
hipError_t launch_reset_states(char* pool, const Shape& sh, const ReqTable& rt, hipStream_t s);

}  // namespace hyf
