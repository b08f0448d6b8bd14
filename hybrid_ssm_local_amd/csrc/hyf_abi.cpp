// libhyflash C ABI: argument validation, state layout, workspace carving and launch order.
// Every host-checkable condition is validated before the first launch, so an error return
// (other than HYF_EHIP) leaves device memory untouched.
#include <string.h>

#include <mutex>

#include "hyf_launch.h"

using namespace hyf;

namespace {

constexpr uint64_t ALIGN = 256;
constexpr int SCAN_TARGET_WGS = 256;         // scan workgroups the segment split aims for (one per CU)
constexpr int64_t SCAN_MIN_SEG_TOKENS = 1024;  // shortest segment the split makes

uint64_t align_up(uint64_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }
int esize(int dtype) { return dtype == HYF_BF16 ? 2 : 4; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_cfg(const hyf_config* c) {
  if (!c) return HYF_EINVAL;
  if (c->dtype != HYF_F32 && c->dtype != HYF_BF16) return HYF_EDTYPE;
  if (c->memory != HYF_MEM_MAMBA2 && c->memory != HYF_MEM_GDN && c->memory != HYF_MEM_LASTW) return HYF_EINVAL;
  if (c->weights != HYF_WEIGHTS_DENSE && c->weights != HYF_WEIGHTS_W4) return HYF_EINVAL;
  if (c->cross_slot != 0 && c->cross_slot != 1) return HYF_EINVAL;
  if (c->d_model < 16 || c->d_model > 65536 || c->d_model % 16) return HYF_ESHAPE;
  if (c->n_heads < 1 || c->n_heads > 1024) return HYF_ESHAPE;
  if (c->head_dim < 16 || c->head_dim > 256 || c->head_dim % 16) return HYF_ESHAPE;
  if (c->d_state < 16 || c->d_state > 256 || c->d_state % 16) return HYF_ESHAPE;
  if (c->n_groups < 1 || c->n_heads % c->n_groups) return HYF_ESHAPE;
  if (c->window < 1 || c->window > 8192) return HYF_ESHAPE;
  if (c->block != HYF_BLOCK) return HYF_ESHAPE;
  if (c->chunk < 16 || c->chunk > 1024 || (c->chunk & (c->chunk - 1))) return HYF_ESHAPE;
  if ((int64_t)c->n_heads * c->head_dim > 65536) return HYF_ESHAPE;
  if (c->weights == HYF_WEIGHTS_W4 &&
      (c->dtype != HYF_BF16 || c->d_model % 128 || ((int64_t)c->n_heads * c->head_dim) % 128))
    return HYF_EUNSUPPORTED;
  return HYF_OK;
}

void fill_layout(const hyf_config* c, hyf_state_layout* L) {
  const uint64_t es = esize(c->dtype);
  L->count_off = 0;
  L->h_off = ALIGN;
  L->k_off = L->h_off + align_up((uint64_t)c->n_heads * c->head_dim * c->d_state * 4);
  const uint64_t ring = align_up((uint64_t)c->n_heads * c->window * c->head_dim * es);
  L->v_off = L->k_off + ring;
  L->total = L->v_off + ring;
  L->b_off = L->dt_off = 0;
  if (c->memory == HYF_MEM_LASTW) {
    L->b_off = L->total;
    L->dt_off = L->b_off + align_up((uint64_t)c->window * c->n_groups * c->d_state * es);
    L->total = L->dt_off + align_up((uint64_t)c->n_heads * c->window * 4);
  }
}

Shape make_shape(const hyf_config* c) {
  Shape s;
  s.d = c->d_model;
  s.nh = c->n_heads;
  s.P = c->head_dim;
  s.N = c->d_state;
  s.G = c->n_groups;
  s.W = c->window;
  s.L = c->chunk;
  s.cross = c->cross_slot;
  s.dq = s.nh * s.P;
  s.gn = s.G * s.N;
  s.off_q = 0;
  s.off_c = s.off_q + s.dq;
  s.off_k = s.off_c + s.gn;
  s.off_v = s.off_k + s.dq;
  s.off_b = s.off_v + s.dq;
  s.off_dt = s.off_b + s.gn;
  s.gdn = c->memory == HYF_MEM_GDN;
  s.w4 = c->weights == HYF_WEIGHTS_W4;
  s.lastw = c->memory == HYF_MEM_LASTW;
  s.off_beta = s.off_dt + s.nh;
  s.n_in = s.off_dt + (s.gdn ? 2 : 1) * s.nh;
  hyf_state_layout L;
  fill_layout(c, &L);
  s.st_bytes = L.total;
  s.st_h = L.h_off;
  s.st_k = L.k_off;
  s.st_v = L.v_off;
  s.st_b = L.b_off;
  s.st_dt = L.dt_off;
  return s;
}


// Segment policy of the scan: whole chunks per segment, the same count for every request, about
// SCAN_TARGET_WGS workgroups in all, segments no shorter than SCAN_MIN_SEG_TOKENS (each segment
// costs one partial state written and read back) and no longer than one workgroup's LDS holds
// weights for.
int64_t scan_seg_target(const Shape& s) {
  const int64_t per_seg = scan_items_per_seg(s);
  const int64_t t = SCAN_TARGET_WGS / per_seg;
  return t < 1 ? 1 : t;
}
int64_t scan_cap_chunks(const Shape& s, int dtype) {
  const int64_t c = scan_max_seg_tokens(s, esize(dtype)) / s.L;
  return c < 1 ? 1 : c;
}
// Segments start on a block boundary of the time-blocked layout: chunks per segment is a
// multiple of HYF_TBLK / L when the chunk is shorter than a block (chunk lengths are powers of 2).
int64_t scan_cps_unit(const Shape& s) { return s.L >= HYF_TBLK ? 1 : HYF_TBLK / s.L; }
int32_t scan_chunks_per_seg(const Shape& s, int dtype, int64_t total_chunks) {
  // One workgroup per CU at a time: the segment count fills whole waves of SCAN_TARGET_WGS
  // workgroups, as many waves as the longest segment LDS allows forces.
  const int64_t unit = scan_cps_unit(s);
  const int64_t cap = scan_cap_chunks(s, dtype) / unit * unit;
  const int64_t per_seg = scan_items_per_seg(s);
  const int64_t need = (total_chunks + cap - 1) / cap;  // segments the cap alone requires
  const int64_t waves = (need * per_seg + SCAN_TARGET_WGS - 1) / SCAN_TARGET_WGS;
  int64_t target = waves * SCAN_TARGET_WGS / per_seg;
  if (target < need) target = need;
  if (target < 1) target = 1;
  int64_t cps = (total_chunks + target - 1) / target;
  const int64_t min_cps = SCAN_MIN_SEG_TOKENS / s.L;
  if (cps < min_cps) cps = min_cps;
  cps = (cps + unit - 1) / unit * unit;
  if (cps > cap) cps = cap;
  return (int32_t)(cps < unit ? unit : cps);
}
// Bound on sum_i ceil(chunks_i / cps): at most (total chunks) / cps + n_req, with total chunks at
// most rows / L + n_req, and (total chunks) / cps at most seg_target unless the cap binds.
int64_t scan_max_segs(const Shape& s, int dtype, int32_t n_req, int64_t rows) {
  const int64_t unit = s.L >= HYF_TBLK ? 1 : HYF_TBLK / s.L;
  int64_t cap = scan_cap_chunks(s, dtype) / unit * unit;
  if (cap < unit) cap = unit;
  return scan_seg_target(s) + 2 * (int64_t)n_req + rows / (cap * s.L) + 3;
}
// y-mode segments are single blocks of HYF_TBLK tokens.
int64_t scan_max_segs_y(int32_t n_req, int64_t rows) { return rows / HYF_TBLK + (int64_t)n_req + 1; }
int64_t scan_segs_bound(const Shape& s, int dtype, int32_t n_req, int64_t rows, bool with_y) {
  const int64_t a = scan_max_segs(s, dtype, n_req, rows);
  const int64_t b = with_y ? scan_max_segs_y(n_req, rows) : 0;
  return a > b ? a : b;
}
// Blocks of the time-blocked buffers for `rows` tokens over R requests (each request starts a block).
int64_t time_blocks(int64_t rows, int32_t R) { return rows / HYF_TBLK + R + 1; }

// Row stride of the round's fp32 projection output: n_in rounded up to 4 floats, so every column
// group starts 16-byte aligned.
int64_t proj_ld(const Shape& s) { return (s.n_in + 3) / 4 * 4; }

// The last-W memory's rescan after a commit (appended to both workspace layouts): every request's
// window as W rows (the first W - min(count, W) of them padding) in the scan's time-blocked
// layout, and the scan's segment partials.
struct WsLastw {
  uint64_t vb, dt, part, lam, end;
};
int64_t lastw_blocks(const Shape& s) { return (s.W + HYF_TBLK - 1) / HYF_TBLK; }
WsLastw ws_lastw(const Shape& s, int dtype, int32_t R, uint64_t base) {
  WsLastw w{};
  uint64_t o = base;
  if (s.lastw) {
    const int64_t nblk = (int64_t)R * lastw_blocks(s);
    const int64_t segs = scan_segs_bound(s, dtype, R, (int64_t)R * s.W, false);
    w.vb = o;
    o += align_up((uint64_t)nblk * (s.dq + s.gn) * HYF_TBLK * esize(dtype));
    w.dt = o;
    o += align_up((uint64_t)nblk * s.nh * HYF_TBLK * 4);
    w.part = o;
    o += align_up((uint64_t)segs * s.nh * s.P * s.N * 4);
    w.lam = o;
    o += align_up((uint64_t)segs * s.nh * 4);
  }
  w.end = o;
  return w;
}

struct WsDraft {
  uint64_t proj, mem, att_part, att_ml, o_in, counters, lastw, end;
};
WsDraft ws_draft(const Shape& s, int dtype, int32_t R, int64_t rows) {
  WsDraft w;
  const int ns = round_max_splits(s);
  uint64_t o = 0;
  w.proj = o;
  o += align_up((uint64_t)(rows + (int64_t)HYF_BLOCK * R) * proj_ld(s) * 4);
  w.mem = o;
  o += align_up((uint64_t)R * HYF_BLOCK * s.dq * 4);
  w.att_part = o;
  o += align_up((uint64_t)R * s.nh * ns * HYF_BLOCK * s.P * 4);
  w.att_ml = o;
  o += align_up((uint64_t)R * s.nh * ns * HYF_BLOCK * 2 * 4);
  w.o_in = o;
  o += align_up((uint64_t)R * HYF_BLOCK * s.dq * esize(dtype));
  w.counters = o;
  o += align_up((uint64_t)(R * s.nh + R) * 4);
  w.lastw = o;
  w.end = ws_lastw(s, dtype, R, o).end;
  return w;
}

struct WsCommit {
  uint64_t vb, dt, kb, c, part, lam, deq, lastw, end;
};
// First w_in row a prefill commit projects through (C for per-token outputs, else k): with 4-bit
// weights the rows from there to n_in are expanded to bf16 in the workspace.
int64_t prefill_row0(const Shape& s) { return s.off_c; }
WsCommit ws_commit(const Shape& s, int dtype, int32_t R, int64_t rows, bool with_y) {
  WsCommit w;
  uint64_t o = 0;
  const int64_t krows = rows < (int64_t)R * s.W ? rows : (int64_t)R * s.W;
  const int64_t segs = scan_segs_bound(s, dtype, R, rows, with_y);
  const int64_t nblk = time_blocks(rows, R);
  w.vb = o;  // v | B time-blocked: [nblk][dq + gn][HYF_TBLK]
  o += align_up((uint64_t)nblk * (s.dq + s.gn) * HYF_TBLK * esize(dtype));
  w.dt = o;  // raw step (or the two raw gates) time-blocked: [nblk][nh or 2 nh][HYF_TBLK] fp32
  o += align_up((uint64_t)nblk * (s.gdn ? 2 : 1) * s.nh * HYF_TBLK * 4);
  w.kb = o;
  o += align_up((uint64_t)krows * s.dq * esize(dtype));
  w.c = o;  // y-mode: C time-blocked: [nblk][gn][HYF_TBLK]
  if (with_y) o += align_up((uint64_t)nblk * s.gn * HYF_TBLK * esize(dtype));
  w.part = o;
  uint64_t part_bytes = (uint64_t)segs * s.nh * s.P * s.N * 4;
  if (s.gdn && gdn_chunked_supported(s, esize(dtype))) {
    // per (chunk of GDN_CHUNK tokens, head) records of the chunked gated delta rule
    const uint64_t chunks = (uint64_t)(rows / GDN_CHUNK + R + 1);
    const uint64_t g = chunks * s.nh * (uint64_t)gdn_chunk_record_floats(s) * 4;
    if (g > part_bytes) part_bytes = g;
  }
  o += align_up(part_bytes);
  w.lam = o;
  o += align_up((uint64_t)segs * s.nh * 4);
  w.deq = o;
  if (s.w4) o += align_up((uint64_t)(s.n_in - prefill_row0(s)) * s.d * 2);
  w.lastw = o;
  w.end = ws_lastw(s, dtype, R, o).end;
  return w;
}

// Request table from host slots / row offsets.  Fills seg0 with the scan's segment split when
// chunks_per_seg > 0.
int build_table(const Shape& s, int32_t pool_slots, const int32_t* slots, int32_t n_req, const int64_t* cu,
                ReqTable* rt) {
  if (n_req < 1 || n_req > HYF_MAX_REQUESTS) return HYF_ECAPACITY;
  memset(rt, 0, sizeof(*rt));
  rt->n_req = n_req;
  for (int i = 0; i < n_req; ++i) {
    const int32_t sl = slots ? slots[i] : i;
    if (sl < 0 || sl >= pool_slots) return HYF_ECAPACITY;
    for (int j = 0; j < i; ++j)
      if (rt->slot[j] == sl) return HYF_EINVAL;  // two requests of one call on one state
    rt->slot[i] = sl;
  }
  if (cu) {
    if (cu[0] != 0) return HYF_EINVAL;
    for (int i = 0; i < n_req; ++i)
      if (cu[i + 1] < cu[i]) return HYF_EINVAL;
    if (cu[n_req] > ((int64_t)1 << 30)) return HYF_ECAPACITY;
    for (int i = 0; i <= n_req; ++i) rt->row0[i] = (int32_t)cu[i];
    int64_t c = 0;
    for (int i = 0; i < n_req; ++i) {
      rt->blk0[i] = (int32_t)c;
      c += (cu[i + 1] - cu[i] + HYF_TBLK - 1) / HYF_TBLK;
    }
    rt->blk0[n_req] = (int32_t)c;
  }
  return HYF_OK;
}

void fill_segments(const Shape& s, int dtype, ReqTable* rt, bool y_mode, int32_t* seg_tokens_out, int32_t* total_out,
                   int32_t* max_out) {
  int32_t seg_tokens = HYF_TBLK;
  if (!y_mode) {
    int64_t total_chunks = 0;
    for (int i = 0; i < rt->n_req; ++i) total_chunks += (rt->row0[i + 1] - rt->row0[i] + s.L - 1) / s.L;
    seg_tokens = scan_chunks_per_seg(s, dtype, total_chunks) * s.L;
  }
  int32_t q = 0, mx = 0;
  for (int i = 0; i < rt->n_req; ++i) {
    rt->seg0[i] = q;
    const int64_t n = rt->row0[i + 1] - rt->row0[i];
    const int32_t ns = (int32_t)((n + seg_tokens - 1) / seg_tokens);
    q += ns;
    if (ns > mx) mx = ns;
  }
  rt->seg0[rt->n_req] = q;
  *seg_tokens_out = seg_tokens;
  *total_out = q;
  *max_out = mx;
}

int hip_status(hipError_t e) { return e == hipSuccess ? HYF_OK : HYF_EHIP; }

int check_weights(const hyf_config* c, const hyf_weights* w) {
  if (!w || !w->a_log || !w->dt_bias || !w->d_skip) return HYF_EINVAL;
  if (c->weights == HYF_WEIGHTS_W4) {
    if (!w->w_in_q || !w->w_in_s || !w->w_out_q || !w->w_out_s) return HYF_EINVAL;
    if (!aligned(w->w_in_q, 16) || !aligned(w->w_out_q, 16) || !aligned(w->w_in_s, 4) || !aligned(w->w_out_s, 4))
      return HYF_EINVAL;
    return HYF_OK;
  }
  if (!w->w_in || !w->w_out) return HYF_EINVAL;
  if (!aligned(w->w_in, 16) || !aligned(w->w_out, 16)) return HYF_EINVAL;
  return HYF_OK;
}

// The layer's input projection restricted to w_in rows row0 .. row0 + n (dense or 4-bit weights).
hipError_t project_in(const Shape& s, int dtype, const hyf_weights* w, int row0, int n, const RowSrc& xs, int64_t M,
                      const Epi& e, hipStream_t hs) {
  if (s.w4)
    return launch_linear_w4_epi(xs, M, s.d, w->w_in_q + (int64_t)row0 * (s.d / 2),
                                w->w_in_s + (int64_t)row0 * (s.d / 128), n, e, hs);
  return launch_linear(dtype, xs, M, s.d, static_cast<const char*>(w->w_in) + (int64_t)row0 * s.d * esize(dtype), n,
                       e, hs);
}
// The layer's output projection.
hipError_t project_out(const Shape& s, int dtype, const hyf_weights* w, const RowSrc& xs, int64_t M, const Epi& e,
                       hipStream_t hs) {
  if (s.w4) return launch_linear_w4_epi(xs, M, s.dq, w->w_out_q, w->w_out_s, s.d, e, hs);
  return launch_linear(dtype, xs, M, s.dq, w->w_out, s.d, e, hs);
}


// The last-W memory after a commit (counts already advanced): every request's window as W rows in
// commit order, padding first (x = 0, so the padding leaves the zero state as it is), into the
// scan's time-blocked layout, H zeroed, then the Mamba-2 scan of those rows into H.
int lastw_rescan(const Shape& s, int dt, const hyf_weights* w, char* pool, const ReqTable& rt_in, char* base,
                 hipStream_t hs) {
  const WsLastw L = ws_lastw(s, dt, rt_in.n_req, 0);
  ReqTable rt = rt_in;
  const int64_t bpr = lastw_blocks(s);
  for (int i = 0; i <= rt.n_req; ++i) {
    rt.row0[i] = (int32_t)((int64_t)i * s.W);
    rt.blk0[i] = (int32_t)((int64_t)i * bpr);
  }
  const int64_t vb_blk = (int64_t)(s.dq + s.gn) * HYF_TBLK, dt_blk = (int64_t)s.nh * HYF_TBLK;
  char* vb = base + L.vb;
  float* dtb = reinterpret_cast<float*>(base + L.dt);
  hipError_t he = launch_lastw_gather(dt, s, pool, rt, vb, vb_blk, dtb, dt_blk, hs);
  if (he != hipSuccess) return HYF_EHIP;
  ScanArgs sa{};
  sa.x = vb;
  sa.B = vb + (int64_t)s.dq * HYF_TBLK * esize(dt);
  sa.dt = dtb;
  sa.xblk = vb_blk;
  sa.bblk = vb_blk;
  sa.dblk = dt_blk;
  sa.a_log = w->a_log;
  sa.dt_bias = w->dt_bias;
  sa.state_pool = pool;
  sa.h_direct = nullptr;
  sa.part = reinterpret_cast<float*>(base + L.part);
  sa.lam = reinterpret_cast<float*>(base + L.lam);
  sa.y_mode = 0;
  sa.d_skip = w->d_skip;
  int32_t max_segs = 0;
  fill_segments(s, dt, &rt, false, &sa.seg_tokens, &sa.total_segs, &max_segs);
  return hip_status(launch_ssd_state(dt, s, sa, rt, max_segs, hs));
}

// Round-sized commit (at most 16 rows per request): one weight pass over the k | v | B | dt rows,
// then one round kernel that folds the rows into H (one read-modify-write), appends them to the
// ring and advances count (the last-W memory: appends them with their B and steps, then rescans).
int commit_round(const hyf_config* cfg, const hyf_weights* w, char* pool, const ReqTable& rt, int64_t rows,
                 const void* feats, char* wsb, hipStream_t hs, const int32_t* dev_rows) {
  const Shape s = make_shape(cfg);
  const int dt = cfg->dtype, n_req = rt.n_req;
  const WsDraft L = ws_draft(s, dt, n_req, rows);
  float* proj = reinterpret_cast<float*>(wsb + L.proj);
  int32_t* counters = reinterpret_cast<int32_t*>(wsb + L.counters);
  const int64_t ld = proj_ld(s);
  RowSrc xs{feats, feats, rows};
  Epi e{proj + s.off_k, ld, 1, s.n_in, nullptr, 0, 0, counters, n_req * s.nh + n_req};
  hipError_t he = project_in(s, dt, w, s.off_k, s.n_in - s.off_k, xs, rows, e, hs);
  if (he != hipSuccess) return HYF_EHIP;
  RoundArgs ra{};
  ra.proj = proj;
  ra.ld = ld;
  ra.blk_row0 = rows;
  ra.state_pool = pool;
  ra.a_log = w->a_log;
  ra.dt_bias = w->dt_bias;
  ra.d_skip = w->d_skip;
  ra.counters = counters;
  ra.do_commit = 1;
  ra.do_draft = 0;
  ra.dev_rows = dev_rows;
  round_layout(s, n_req, esize(dt), &ra);
  ra.n_split = 0;
  if ((he = launch_round(dt, s, ra, rt, hs)) != hipSuccess) return HYF_EHIP;
  if (s.lastw) return lastw_rescan(s, dt, w, pool, rt, wsb + L.lastw, hs);
  return HYF_OK;
}

// Host checks of a draft call (everything but the workspace); fills the request table and the
// number of commit rows.
int draft_check(const hyf_config* cfg, const hyf_weights* w, void* state_pool, int32_t pool_slots,
                const int32_t* slots, int32_t n_req, const void* commit_feats, const int64_t* cu_commit,
                const void* block_in, void* block_out, ReqTable* rt, int64_t* rows_out) {
  int st = check_cfg(cfg);
  if (st != HYF_OK) return st;
  if ((st = check_weights(cfg, w)) != HYF_OK) return st;
  if (!state_pool || !aligned(state_pool, ALIGN) || pool_slots < 1) return HYF_EINVAL;
  if (!block_in || !block_out || !aligned(block_in, 16) || !aligned(block_out, 16)) return HYF_EINVAL;
  if ((commit_feats == nullptr) != (cu_commit == nullptr)) return HYF_EINVAL;
  const Shape s = make_shape(cfg);
  if ((st = build_table(s, pool_slots, slots, n_req, cu_commit, rt)) != HYF_OK) return st;
  int64_t rows = 0;
  if (cu_commit) {
    rows = cu_commit[n_req];
    for (int i = 0; i < n_req; ++i)
      if (cu_commit[i + 1] - cu_commit[i] > HYF_BLOCK) return HYF_ECAPACITY;
    if (rows > 0 && !aligned(commit_feats, 16)) return HYF_EINVAL;
  }
  *rows_out = rows;
  return HYF_OK;
}

// The launches of a draft call, after every check has passed: ws holds at least
// hyf_workspace_bytes(cfg, n_req, rows, 0) bytes, 256-byte aligned.
int draft_run(const hyf_config* cfg, const hyf_weights* w, void* state_pool, const ReqTable& rt, int64_t rows,
              const void* commit_feats, const void* block_in, void* block_out, char* wsb, hipStream_t hs,
              const int32_t* dev_rows) {
  const Shape s = make_shape(cfg);
  const int n_req = rt.n_req;
  char* pool = static_cast<char*>(state_pool);
  const int dt = cfg->dtype;
  if (s.lastw && rows > 0) {
    // the window's scan has to follow the append: commit, then draft without commit rows
    const int st = commit_round(cfg, w, pool, rt, rows, commit_feats, wsb, hs, dev_rows);
    if (st != HYF_OK) return st;
    rows = 0;
    dev_rows = nullptr;
  }
  const WsDraft L = ws_draft(s, dt, n_req, rows);
  float* proj = reinterpret_cast<float*>(wsb + L.proj);

  // 1. one pass over w_in for [commit rows ; block rows] (it also clears the round's counters)
  int32_t* counters = reinterpret_cast<int32_t*>(wsb + L.counters);
  const int64_t ld = proj_ld(s);
  RowSrc xs{rows > 0 ? commit_feats : block_in, block_in, rows};
  Epi e{proj, ld, 1, s.n_in, nullptr, 0, 0, counters, n_req * s.nh + n_req};
  hipError_t he = project_in(s, dt, w, 0, s.n_in, xs, rows + (int64_t)HYF_BLOCK * n_req, e, hs);
  if (he != hipSuccess) return HYF_EHIP;

  // 2. the round kernel: commit + readout tiles and attention splits, merged per head
  RoundArgs ra{};
  ra.proj = proj;
  ra.ld = ld;
  ra.blk_row0 = rows;
  ra.state_pool = pool;
  ra.a_log = w->a_log;
  ra.dt_bias = w->dt_bias;
  ra.d_skip = w->d_skip;
  ra.mem = reinterpret_cast<float*>(wsb + L.mem);
  ra.att_part = reinterpret_cast<float*>(wsb + L.att_part);
  ra.att_ml = reinterpret_cast<float*>(wsb + L.att_ml);
  ra.o_in = wsb + L.o_in;
  ra.counters = counters;
  ra.do_commit = rows > 0;
  ra.do_draft = 1;
  ra.dev_rows = dev_rows;
  round_layout(s, n_req, esize(dt), &ra);
  if ((he = launch_round(dt, s, ra, rt, hs)) != hipSuccess) return HYF_EHIP;
  // 3. output projection
  RowSrc xo{ra.o_in, ra.o_in, (int64_t)HYF_BLOCK * n_req};
  Epi eo{block_out, s.d, 0, s.d, nullptr, 0, 0, nullptr, 0};
  return hip_status(project_out(s, dt, w, xo, (int64_t)HYF_BLOCK * n_req, eo, hs));
}

// ---- the allocation-free draft call's scratch --------------------------------------------------
// One array per GPU, in the library's code object: each device that loads the library holds its own
// copy until the process ends.  Host code never uses the array's name as an address (on the host it
// names a stand-in, not device memory): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and is kept per device.  Every call on one device
// shares its array, so overlapping calls on one device race.
static __device__ __align__(256) unsigned char scratch[HYF_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

int noalloc_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return HYF_EHIP;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return HYF_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HYF_EHIP;
    if (!aligned(p, ALIGN)) return HYF_EHIP;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return HYF_OK;
}

}  // namespace

extern "C" {

int hyf_abi_version(void) { return HYF_ABI_VERSION; }

const char* hyf_status_str(int st) {
  switch (st) {
    case HYF_OK: return "ok";
    case HYF_EINVAL: return "invalid argument";
    case HYF_ESHAPE: return "unsupported or inconsistent shape";
    case HYF_ECAPACITY: return "capacity exceeded";
    case HYF_EDTYPE: return "unknown dtype";
    case HYF_EWORKSPACE: return "workspace too small";
    case HYF_EUNSUPPORTED: return "mode not implemented";
    case HYF_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int hyf_config_check(const hyf_config* cfg) { return check_cfg(cfg); }

int64_t hyf_n_in(const hyf_config* cfg) {
  if (check_cfg(cfg) != HYF_OK) return 0;
  return make_shape(cfg).n_in;
}

int hyf_state_layout_get(const hyf_config* cfg, hyf_state_layout* out) {
  const int st = check_cfg(cfg);
  if (st != HYF_OK) return st;
  if (!out) return HYF_EINVAL;
  fill_layout(cfg, out);
  return HYF_OK;
}

size_t hyf_state_bytes(const hyf_config* cfg) {
  if (check_cfg(cfg) != HYF_OK) return 0;
  hyf_state_layout L;
  fill_layout(cfg, &L);
  return (size_t)L.total;
}

size_t hyf_workspace_bytes(const hyf_config* cfg, int32_t max_requests, int64_t max_rows, int32_t with_y) {
  if (check_cfg(cfg) != HYF_OK || max_requests < 1 || max_requests > HYF_MAX_REQUESTS || max_rows < 0) return 0;
  const Shape s = make_shape(cfg);
  // the draft-sized layout serves draft calls (at most HYF_BLOCK commit rows per request) and round-sized
  // commits (at most RMAXC rows per request); longer commits take the commit layout
  const int64_t round_rows = (int64_t)16 * max_requests;
  const uint64_t a = ws_draft(s, cfg->dtype, max_requests, max_rows < round_rows ? max_rows : round_rows).end;
  const uint64_t b = ws_commit(s, cfg->dtype, max_requests, max_rows, with_y != 0).end;
  return (size_t)(a > b ? a : b);
}

size_t hyf_ssd_scan_workspace_bytes(const hyf_config* cfg, int64_t T, int32_t with_y) {
  if (check_cfg(cfg) != HYF_OK || T < 0) return 0;
  const Shape s = make_shape(cfg);
  const int64_t segs = scan_segs_bound(s, cfg->dtype, 1, T, with_y != 0);
  return (size_t)(align_up((uint64_t)segs * s.nh * s.P * s.N * 4) + align_up((uint64_t)segs * s.nh * 4));
}

int hyf_state_reset(const hyf_config* cfg, void* state_pool, int32_t pool_slots, const int32_t* slots, int32_t n_req,
                    void* stream) {
  int st = check_cfg(cfg);
  if (st != HYF_OK) return st;
  if (!state_pool || !aligned(state_pool, ALIGN) || pool_slots < 1) return HYF_EINVAL;
  const Shape s = make_shape(cfg);
  ReqTable rt;
  st = build_table(s, pool_slots, slots, n_req, nullptr, &rt);
  if (st != HYF_OK) return st;
  return hip_status(launch_reset_states(static_cast<char*>(state_pool), s, rt, static_cast<hipStream_t>(stream)));
}

int hyf_memory_commit(const hyf_config* cfg, const hyf_weights* w, void* state_pool, int32_t pool_slots,
                      const int32_t* slots, int32_t n_req, const void* feats, const int64_t* cu_rows, void* y_opt,
                      void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != HYF_OK) return st;
  if ((st = check_weights(cfg, w)) != HYF_OK) return st;
  if (!state_pool || !aligned(state_pool, ALIGN) || pool_slots < 1 || !cu_rows) return HYF_EINVAL;
  const Shape s = make_shape(cfg);
  if (y_opt && (s.gdn || s.lastw || !scan_y_supported(s, esize(cfg->dtype)))) return HYF_EUNSUPPORTED;
  if (y_opt && !aligned(y_opt, 16)) return HYF_EINVAL;
  ReqTable rt;
  if ((st = build_table(s, pool_slots, slots, n_req, cu_rows, &rt)) != HYF_OK) return st;
  const int64_t rows = cu_rows[n_req];
  if (rows == 0) return HYF_OK;
  if (!feats || !aligned(feats, 16)) return HYF_EINVAL;
  if (!ws || !aligned(ws, ALIGN) || ws_bytes < hyf_workspace_bytes(cfg, n_req, rows, y_opt != nullptr))
    return HYF_EWORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  char* pool = static_cast<char*>(state_pool);
  const int dt = cfg->dtype;
  const int es = esize(dt);

  int64_t max_n = 0;
  for (int i = 0; i < n_req; ++i) max_n = cu_rows[i + 1] - cu_rows[i] > max_n ? cu_rows[i + 1] - cu_rows[i] : max_n;

  // a gated delta-rule prefix takes the chunked kernels when they fit the shape, else the
  // token-by-token one; refused only when neither fits
  if (s.gdn && max_n > 16 && !gdn_supported(s) && !gdn_chunked_supported(s, es)) return HYF_EUNSUPPORTED;
  if (max_n <= 16 && !y_opt) return commit_round(cfg, w, pool, rt, rows, feats, wsb, hs, nullptr);

  // Prefill-sized commit (or any commit with per-token outputs): projection GEMMs -> ring append ->
  // scan -> count.  The GEMM epilogues write the scan's operands time-blocked (each request's
  // tokens start a block): v and B (and C for y) tiled for the scan's MFMA fragments, dt plain.
  const bool with_y = y_opt != nullptr;
  const WsCommit L = ws_commit(s, dt, n_req, rows, with_y);
  char* cT = wsb + L.c;
  const int64_t c_blk = (int64_t)s.gn * HYF_TBLK;
  hipError_t he;
  // the w_in rows from prefill_row0 on, dense: the caller's, or (4-bit weights) expanded to bf16
  const char* w_rows = static_cast<const char*>(w->w_in) + prefill_row0(s) * (int64_t)s.d * es;
  if (s.w4) {
    char* deq = wsb + L.deq;
    const int64_t r0 = prefill_row0(s);
    if ((he = launch_w4_dequant(w->w_in_q + r0 * (s.d / 2), w->w_in_s + r0 * (s.d / 128), (int)(s.n_in - r0), s.d,
                                reinterpret_cast<bf16*>(deq), hs)) != hipSuccess)
      return HYF_EHIP;
    w_rows = deq;
  }
  auto w_row = [&](int r) { return w_rows + (int64_t)(r - prefill_row0(s)) * s.d * es; };
  const char* w_c = w_row(s.off_c);
  char* vbT = wsb + L.vb;
  float* dtT = reinterpret_cast<float*>(wsb + L.dt);
  char* kb = wsb + L.kb;
  const int nvb = s.dq + s.gn;
  const int64_t vb_blk = (int64_t)nvb * HYF_TBLK;  // block strides (elements) of v | B and of dt
  const int ndt = (s.gdn ? 2 : 1) * s.nh;  // raw step, or the two raw gates
  const int64_t dt_blk = (int64_t)ndt * HYF_TBLK;
  const char* w_vbd = w_row(s.off_v);
  const char* w_k = w_row(s.off_k);
  int64_t krow = 0;
  if (dt == HYF_BF16 && s.d % 64 == 0) {
    // bf16: one grouped GEMM launch over every request's rows for v | B | dt (and C), one for k
    // (each request's last min(n_i, W) rows).  Each request's time-blocked output starts its own
    // block, so its product rows start on a multiple of 8 (padding rows between requests); the k
    // rows are row-major and packed.
    RowGroups gv{}, gk{};
    gv.n = gk.n = n_req;
    gv.m0[0] = gk.m0[0] = 0;
    for (int i = 0; i < n_req; ++i) {
      const int64_t n = cu_rows[i + 1] - cu_rows[i];
      const int64_t m = n < s.W ? n : s.W;
      gv.m0[i + 1] = (int32_t)(gv.m0[i] + (n + 7) / 8 * 8);
      gv.cnt[i] = (int32_t)n;
      gv.src0[i] = (int32_t)cu_rows[i];
      gv.blk0[i] = rt.blk0[i];
      gk.m0[i + 1] = (int32_t)(gk.m0[i] + m);
      gk.cnt[i] = (int32_t)m;
      gk.src0[i] = (int32_t)(cu_rows[i + 1] - m);
      gk.blk0[i] = 0;
    }
    const bf16* X = static_cast<const bf16*>(feats);
    Epi e{vbT, vb_blk, 0, nvb, dtT, dt_blk, 1};
    if ((he = launch_gemm_grouped(X, gv, s.d, reinterpret_cast<const bf16*>(w_vbd), nvb + ndt, e, hs)) != hipSuccess)
      return HYF_EHIP;
    if (with_y) {
      Epi ec{cT, c_blk, 0, s.gn, nullptr, 0, 1};
      if ((he = launch_gemm_grouped(X, gv, s.d, reinterpret_cast<const bf16*>(w_c), s.gn, ec, hs)) != hipSuccess)
        return HYF_EHIP;
    }
    Epi ek{kb, s.dq, 0, s.dq, nullptr, 0, 0};
    if ((he = launch_gemm_grouped(X, gk, s.d, reinterpret_cast<const bf16*>(w_k), s.dq, ek, hs)) != hipSuccess)
      return HYF_EHIP;
  }
  for (int i = 0; i < n_req && !(dt == HYF_BF16 && s.d % 64 == 0); ++i) {
    const int64_t n = cu_rows[i + 1] - cu_rows[i];
    if (n == 0) continue;
    const char* src = static_cast<const char*>(feats) + cu_rows[i] * (int64_t)s.d * es;
    RowSrc xs{src, src, n};
    Epi e{vbT + rt.blk0[i] * vb_blk * es, vb_blk, 0, nvb, dtT + rt.blk0[i] * dt_blk, dt_blk, 1};
    if ((he = launch_linear(dt, xs, n, s.d, w_vbd, nvb + ndt, e, hs)) != hipSuccess) return HYF_EHIP;
    if (with_y) {
      Epi ec{cT + rt.blk0[i] * c_blk * es, c_blk, 0, s.gn, nullptr, 0, 1};
      if ((he = launch_linear(dt, xs, n, s.d, w_c, s.gn, ec, hs)) != hipSuccess) return HYF_EHIP;
    }
    // k only for the rows that stay in the window: the last min(n_i, W) of the request.
    const int64_t m = n < s.W ? n : s.W;
    const char* ksrc = src + (n - m) * (int64_t)s.d * es;
    RowSrc ks{ksrc, ksrc, m};
    Epi ek{kb + krow * s.dq * es, s.dq, 0, s.dq, nullptr, 0, 0};
    if ((he = launch_linear(dt, ks, m, s.d, w_k, s.dq, ek, hs)) != hipSuccess) return HYF_EHIP;
    krow += m;
  }
  if ((he = launch_ring_append(dt, s, pool, rt, kb, s.dq, vbT, vb_blk, dtT, dt_blk, hs)) != hipSuccess)
    return HYF_EHIP;
  ScanArgs sa{};
  sa.x = vbT;
  sa.B = vbT + (int64_t)s.dq * HYF_TBLK * es;
  sa.dt = dtT;
  sa.xblk = vb_blk;
  sa.bblk = vb_blk;
  sa.dblk = dt_blk;
  sa.a_log = w->a_log;
  sa.dt_bias = w->dt_bias;
  sa.state_pool = pool;
  sa.h_direct = nullptr;
  sa.part = reinterpret_cast<float*>(wsb + L.part);
  sa.lam = reinterpret_cast<float*>(wsb + L.lam);
  sa.y_mode = with_y;
  sa.C = cT;
  sa.cblk = c_blk;
  sa.y = y_opt;
  sa.d_skip = w->d_skip;
  if (s.lastw) {
    // the last-W memory keeps no running fold: the rings now hold the window; rescan it
    if ((he = launch_bump_counts(pool, s, rt, hs)) != hipSuccess) return HYF_EHIP;
    return lastw_rescan(s, dt, w, pool, rt, wsb + L.lastw, hs);
  }
  if (s.gdn) {
    // chunk offsets of the chunked form (unused by the token-by-token kernel)
    int32_t q = 0;
    for (int i = 0; i < rt.n_req; ++i) {
      rt.seg0[i] = q;
      q += (int32_t)((rt.row0[i + 1] - rt.row0[i] + GDN_CHUNK - 1) / GDN_CHUNK);
    }
    rt.seg0[rt.n_req] = q;
    he = launch_gdn_commit(dt, s, sa, rt, hs);
  } else {
    int32_t max_segs = 0;
    fill_segments(s, dt, &rt, with_y, &sa.seg_tokens, &sa.total_segs, &max_segs);
    he = launch_ssd_state(dt, s, sa, rt, max_segs, hs);
  }
  if (he != hipSuccess) return HYF_EHIP;
  return hip_status(launch_bump_counts(pool, s, rt, hs));
}

int hyf_draft_block(const hyf_config* cfg, const hyf_weights* w, void* state_pool, int32_t pool_slots,
                    const int32_t* slots, int32_t n_req, const void* commit_feats, const int64_t* cu_commit,
                    const void* block_in, void* block_out, void* ws, size_t ws_bytes, void* stream) {
  ReqTable rt;
  int64_t rows = 0;
  int st = draft_check(cfg, w, state_pool, pool_slots, slots, n_req, commit_feats, cu_commit, block_in, block_out,
                       &rt, &rows);
  if (st != HYF_OK) return st;
  if (!ws || !aligned(ws, ALIGN) || ws_bytes < hyf_workspace_bytes(cfg, n_req, rows, 0)) return HYF_EWORKSPACE;
  return draft_run(cfg, w, state_pool, rt, rows, commit_feats, block_in, block_out, static_cast<char*>(ws),
                   static_cast<hipStream_t>(stream), nullptr);
}

int hyf_draft_block_noalloc(const hyf_config* cfg, const hyf_weights* w, void* state_pool, int32_t pool_slots,
                            const int32_t* slots, int32_t n_req, const void* commit_feats, const int64_t* cu_commit,
                            const void* block_in, void* block_out, void* stream) {
  ReqTable rt;
  int64_t rows = 0;
  int st = draft_check(cfg, w, state_pool, pool_slots, slots, n_req, commit_feats, cu_commit, block_in, block_out,
                       &rt, &rows);
  if (st != HYF_OK) return st;
  // a draft call uses only the draft part of the workspace hyf_workspace_bytes sizes
  if (ws_draft(make_shape(cfg), cfg->dtype, n_req, rows).end > (uint64_t)HYF_NOALLOC_SCRATCH_BYTES)
    return HYF_ECAPACITY;
  char* ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != HYF_OK) return st;
  return draft_run(cfg, w, state_pool, rt, rows, commit_feats, block_in, block_out, ws,
                   static_cast<hipStream_t>(stream), nullptr);
}

int hyf_draft_block_dev(const hyf_config* cfg, const hyf_weights* w, void* state_pool, int32_t pool_slots,
                        const int32_t* slots, int32_t n_req, const void* commit_feats, const int32_t* commit_rows,
                        const void* block_in, void* block_out, void* ws, size_t ws_bytes, void* stream) {
  // the host checks of hyf_draft_block with a table of HYF_BLOCK padded commit rows per request
  // (their real counts come from commit_rows on the device)
  if (n_req < 0 || n_req > HYF_MAX_REQUESTS) return HYF_EINVAL;
  if ((commit_feats == nullptr) != (commit_rows == nullptr)) return HYF_EINVAL;
  if (commit_rows && !aligned(commit_rows, 4)) return HYF_EINVAL;
  int64_t cu[HYF_MAX_REQUESTS + 1];
  for (int i = 0; i <= n_req; ++i) cu[i] = commit_feats ? (int64_t)HYF_BLOCK * i : 0;
  ReqTable rt;
  int64_t rows = 0;
  int st = draft_check(cfg, w, state_pool, pool_slots, slots, n_req, commit_feats, commit_feats ? cu : nullptr,
                       block_in, block_out, &rt, &rows);
  if (st != HYF_OK) return st;
  if (!ws || !aligned(ws, ALIGN) || ws_bytes < hyf_workspace_bytes(cfg, n_req, rows, 0)) return HYF_EWORKSPACE;
  return draft_run(cfg, w, state_pool, rt, rows, commit_feats, block_in, block_out, static_cast<char*>(ws),
                   static_cast<hipStream_t>(stream), rows > 0 ? commit_rows : nullptr);
}

int hyf_linear(const hyf_config* cfg, const void* X, int64_t M, int32_t K, const void* W, int32_t Nout, void* out,
               int32_t out_f32, void* stream) {
  const int st = check_cfg(cfg);
  if (st != HYF_OK) return st;
  if (M < 0 || M > ((int64_t)1 << 30) || K < 8 || K % 8 || Nout < 1) return HYF_ESHAPE;
  if (M == 0) return HYF_OK;
  if (!X || !W || !out || !aligned(X, 16) || !aligned(W, 16) || !aligned(out, 4)) return HYF_EINVAL;
  RowSrc xs{X, X, M};
  Epi e{out, Nout, out_f32 ? 1 : 0, Nout, nullptr, 0};
  return hip_status(launch_linear(cfg->dtype, xs, M, K, W, Nout, e, static_cast<hipStream_t>(stream)));
}

int hyf_linear_w4(const hyf_config* cfg, const void* X, int64_t M, int32_t K, const void* Wq, const float* scales,
                  int32_t Nout, void* out, int32_t out_f32, void* stream) {
  const int st = check_cfg(cfg);
  if (st != HYF_OK) return st;
  if (cfg->dtype != HYF_BF16) return HYF_EUNSUPPORTED;
  if (M < 0 || M > (int64_t)64 * 65535 || K < 128 || K % 128 || Nout < 1 || Nout > (1 << 24)) return HYF_ESHAPE;
  if (M == 0) return HYF_OK;
  if (!X || !Wq || !scales || !out || !aligned(X, 16) || !aligned(Wq, 16) || !aligned(scales, 4) ||
      !aligned(out, out_f32 ? 4 : 2))
    return HYF_EINVAL;
  return hip_status(launch_linear_w4(static_cast<const bf16*>(X), M, K, static_cast<const uint8_t*>(Wq), scales,
                                     Nout, out, out_f32 != 0, static_cast<hipStream_t>(stream)));
}

int hyf_ssd_scan(const hyf_config* cfg, const void* x, const void* B, const void* C_opt, const float* dt_raw,
                 const float* a_log, const float* dt_bias, const float* d_skip, float* H_inout, void* y_opt, int64_t T,
                 void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != HYF_OK) return st;
  if (T < 0 || T > ((int64_t)1 << 30)) return HYF_ECAPACITY;
  if (!a_log || !dt_bias || !d_skip || !H_inout || !aligned(H_inout, 16)) return HYF_EINVAL;
  if ((y_opt != nullptr) != (C_opt != nullptr)) return HYF_EINVAL;
  const Shape s = make_shape(cfg);
  if (s.gdn) return HYF_EUNSUPPORTED;  // the scan on pre-projected inputs is the Mamba-2 memory's
  if (y_opt && !scan_y_supported(s, esize(cfg->dtype))) return HYF_EUNSUPPORTED;
  if (T == 0) return HYF_OK;
  if (!x || !B || !dt_raw || !aligned(x, 16) || !aligned(B, 16) || !aligned(dt_raw, 16)) return HYF_EINVAL;
  if (y_opt && (!aligned(C_opt, 16) || !aligned(y_opt, 16))) return HYF_EINVAL;
  if (!ws || !aligned(ws, ALIGN) || ws_bytes < hyf_ssd_scan_workspace_bytes(cfg, T, y_opt != nullptr))
    return HYF_EWORKSPACE;
  ReqTable rt;
  memset(&rt, 0, sizeof(rt));
  rt.n_req = 1;
  rt.row0[1] = (int32_t)T;
  rt.blk0[1] = (int32_t)((T + HYF_TBLK - 1) / HYF_TBLK);
  ScanArgs sa{};
  sa.x = x;
  sa.B = B;
  sa.dt = dt_raw;
  sa.xblk = (int64_t)s.nh * s.P * HYF_TBLK;
  sa.bblk = (int64_t)s.gn * HYF_TBLK;
  sa.dblk = (int64_t)s.nh * HYF_TBLK;
  sa.a_log = a_log;
  sa.dt_bias = dt_bias;
  sa.state_pool = nullptr;
  sa.h_direct = H_inout;
  const int64_t segs = scan_segs_bound(s, cfg->dtype, 1, T, y_opt != nullptr);
  sa.part = static_cast<float*>(ws);
  sa.lam = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((uint64_t)segs * s.nh * s.P * s.N * 4));
  sa.y_mode = y_opt != nullptr;
  sa.C = C_opt;
  sa.cblk = (int64_t)s.gn * HYF_TBLK;
  sa.y = y_opt;
  sa.d_skip = d_skip;
  int32_t max_segs = 0;
  fill_segments(s, cfg->dtype, &rt, y_opt != nullptr, &sa.seg_tokens, &sa.total_segs, &max_segs);
  return hip_status(launch_ssd_state(cfg->dtype, s, sa, rt, max_segs, static_cast<hipStream_t>(stream)));
}

// ---- the full drafter block ----------------------------------------------------------------

namespace {

int check_block(const hyf_config* cfg, const hyf_block_weights* bw) {
  if (!bw || !bw->norm1 || !bw->norm2 || !bw->w_gate_up || !bw->w_down) return HYF_EINVAL;
  if (!aligned(bw->norm1, 16) || !aligned(bw->norm2, 16) || !aligned(bw->w_gate_up, 16) || !aligned(bw->w_down, 16))
    return HYF_EINVAL;
  if (bw->d_ff < 16 || bw->d_ff % 16 != 0 || !(bw->eps >= 0.f) || bw->eps > 1.f) return HYF_ESHAPE;
  (void)cfg;
  return HYF_OK;
}

// Block workspace: the layer's own workspace first, then the block's buffers for up to `rows`
// committed rows and R blocks: normalized commit rows and block rows (storage dtype), the
// layer's output (storage dtype), h (fp32), z (storage dtype), gate|up (fp32), the gated
// product (storage dtype) and the down projection (fp32).
struct WsBlock {
  uint64_t inner, xc, xb, o, h, z, gu, a, y, end;
};
WsBlock ws_block(const hyf_config* cfg, const hyf_block_weights* bw, int32_t R, int64_t rows) {
  WsBlock L{};
  const uint64_t es = esize(cfg->dtype), d = cfg->d_model, F = bw->d_ff, nb = (uint64_t)HYF_BLOCK * R;
  uint64_t o = align_up(hyf_workspace_bytes(cfg, R, rows, 0));
  L.inner = 0;
  L.xc = o; o += align_up((uint64_t)rows * d * es);
  L.xb = o; o += align_up(nb * d * es);
  L.o = o; o += align_up(nb * d * es);
  L.h = o; o += align_up(nb * d * 4);
  L.z = o; o += align_up(nb * d * es);
  L.gu = o; o += align_up(nb * 2 * F * 4);
  L.a = o; o += align_up(nb * F * es);
  L.y = o; o += align_up(nb * d * 4);
  L.end = o;
  return L;
}

}  // namespace

size_t hyf_block_workspace_bytes(const hyf_config* cfg, const hyf_block_weights* bw, int32_t max_requests,
                                 int64_t max_rows) {
  if (check_cfg(cfg) != HYF_OK || check_block(cfg, bw) != HYF_OK || max_requests < 1 ||
      max_requests > HYF_MAX_REQUESTS || max_rows < 0)
    return 0;
  return (size_t)ws_block(cfg, bw, max_requests, max_rows).end;
}

int hyf_block_commit(const hyf_config* cfg, const hyf_weights* w, const hyf_block_weights* bw, void* state_pool,
                     int32_t pool_slots, const int32_t* slots, int32_t n_req, const void* feats,
                     const int64_t* cu_rows, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != HYF_OK) return st;
  if ((st = check_block(cfg, bw)) != HYF_OK) return st;
  if (n_req < 0 || n_req > HYF_MAX_REQUESTS || !cu_rows) return HYF_EINVAL;
  if (n_req == 0) return hyf_memory_commit(cfg, w, state_pool, pool_slots, slots, n_req, feats, cu_rows, nullptr, ws,
                                           ws_bytes, stream);
  const int64_t rows = cu_rows[n_req];
  if (rows < 0) return HYF_EINVAL;
  if (rows > 0 && (!feats || !aligned(feats, 16))) return HYF_EINVAL;
  if (!ws || !aligned(ws, ALIGN) || ws_bytes < hyf_block_workspace_bytes(cfg, bw, n_req, rows)) return HYF_EWORKSPACE;
  const WsBlock L = ws_block(cfg, bw, n_req, rows);
  char* wsb = static_cast<char*>(ws);
  // the layer's checks (weights, state, table) run before anything is launched
  const Shape s = make_shape(cfg);
  ReqTable rt;
  if ((st = check_weights(cfg, w)) != HYF_OK) return st;
  if (!state_pool || !aligned(state_pool, ALIGN) || pool_slots < 1) return HYF_EINVAL;
  if ((st = build_table(s, pool_slots, slots, n_req, cu_rows, &rt)) != HYF_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (launch_rmsnorm(cfg->dtype, feats, rows, cfg->d_model, bw->norm1, bw->eps, wsb + L.xc, hs) != hipSuccess)
    return HYF_EHIP;
  return hyf_memory_commit(cfg, w, state_pool, pool_slots, slots, n_req, rows > 0 ? wsb + L.xc : feats, cu_rows,
                           nullptr, wsb + L.inner, hyf_workspace_bytes(cfg, n_req, rows, 0), stream);
}

int hyf_block_draft(const hyf_config* cfg, const hyf_weights* w, const hyf_block_weights* bw, void* state_pool,
                    int32_t pool_slots, const int32_t* slots, int32_t n_req, const void* commit_feats,
                    const int64_t* cu_commit, const void* block_in, void* block_out, void* ws, size_t ws_bytes,
                    void* stream) {
  ReqTable rt;
  int64_t rows = 0;
  int st = draft_check(cfg, w, state_pool, pool_slots, slots, n_req, commit_feats, cu_commit, block_in, block_out,
                       &rt, &rows);
  if (st != HYF_OK) return st;
  if ((st = check_block(cfg, bw)) != HYF_OK) return st;
  if (!ws || !aligned(ws, ALIGN) || ws_bytes < hyf_block_workspace_bytes(cfg, bw, n_req, rows)) return HYF_EWORKSPACE;
  const int64_t nbytes_in = (int64_t)HYF_BLOCK * n_req * cfg->d_model * esize(cfg->dtype);
  const char* bi = static_cast<const char*>(block_in);
  const char* bo = static_cast<const char*>(block_out);
  if (bi < bo + nbytes_in && bo < bi + nbytes_in) return HYF_EINVAL;  // block_out overlaps block_in
  const WsBlock L = ws_block(cfg, bw, n_req, rows);
  char* wsb = static_cast<char*>(ws);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int dt = cfg->dtype, d = cfg->d_model, F = bw->d_ff;
  const int64_t nb = (int64_t)HYF_BLOCK * n_req;
  hipError_t he;
  // the layer reads its own inputs: the normalized commit rows and block rows
  if (rows > 0 && (he = launch_rmsnorm(dt, commit_feats, rows, d, bw->norm1, bw->eps, wsb + L.xc, hs)) != hipSuccess)
    return HYF_EHIP;
  if ((he = launch_rmsnorm(dt, block_in, nb, d, bw->norm1, bw->eps, wsb + L.xb, hs)) != hipSuccess) return HYF_EHIP;
  if ((st = draft_run(cfg, w, state_pool, rt, rows, rows > 0 ? wsb + L.xc : nullptr, wsb + L.xb, wsb + L.o,
                      wsb + L.inner, hs, nullptr)) != HYF_OK)
    return st;
  // h = x + o, z = RMSNorm(h) norm2; gate|up = z w_gate_up^T; a = silu(gate) up; y = a w_down^T; out = h + y
  float* h = reinterpret_cast<float*>(wsb + L.h);
  float* gu = reinterpret_cast<float*>(wsb + L.gu);
  float* y = reinterpret_cast<float*>(wsb + L.y);
  if ((he = launch_resid_norm(dt, block_in, wsb + L.o, nb, d, bw->norm2, bw->eps, h, wsb + L.z, hs)) != hipSuccess)
    return HYF_EHIP;
  Epi e1{gu, 2 * (int64_t)F, 1, 2 * F, nullptr, 0, 0};
  if ((he = launch_linear(dt, RowSrc{wsb + L.z, wsb + L.z, nb}, nb, d, bw->w_gate_up, 2 * F, e1, hs)) != hipSuccess)
    return HYF_EHIP;
  if ((he = launch_swiglu(dt, gu, nb, F, wsb + L.a, hs)) != hipSuccess) return HYF_EHIP;
  Epi e2{y, (int64_t)d, 1, d, nullptr, 0, 0};
  if ((he = launch_linear(dt, RowSrc{wsb + L.a, wsb + L.a, nb}, nb, F, bw->w_down, d, e2, hs)) != hipSuccess)
    return HYF_EHIP;
  return hip_status(launch_add_out(dt, h, y, nb * d, block_out, hs));
}

}  // extern "C"
