// Engine of layer-skip self-speculative greedy decoding on one gfx950 GPU,
// and its C ABI (include/lss.h).
//
// One forward code path serves every row block: prefill chunks, draft steps
// (one row, skip mask, optional int8 activations), verify (k + 1 causal
// rows), the autoregressive baseline (verify of one row) and the CLaSp
// layer-selection rows (all at one position, each seeing the committed prefix
// plus its own key/value).  Because every kernel is row-independent with a
// fixed reduction order, verify rows equal autoregressive steps bit for bit.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <array>
#include <mutex>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/lss.h"
#include "lss_kernels.h"
#include "lss_router.h"

using namespace lss;

namespace {

constexpr int kWinMax = LSS_WINDOW_MAX;
#define LSS_MAX_DEVICES 64

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// K splits of a prefill / layer-selection GEMM (measured at the 8B shapes):
// wide N keeps ~512 workgroups with few splits (each split adds a pass of
// the epilogue), narrow N splits up to 8 ways to reach ~1024 workgroups; at
// least 4 steps of K per split
int pg_splits(int N, int K, int wbytes) {
  const int KS = wbytes == 2 ? 128 : 64;
  const int nsteps = (K + KS - 1) / KS;
  const int tiles = (N + PG_TN - 1) / PG_TN;
  int S = tiles >= 128 ? 512 / tiles : (1024 + tiles - 1) / tiles;
  S = std::min(S, std::max(1, nsteps / 4));
  return std::max(1, std::min(S, PG_MAX_SPLIT));
}

// token slots per sequence (pending token + window)
constexpr int kTokSlots = 64;

struct Layout {
  size_t seq_kv;   // bytes of one sequence's K (or V) cache
  int nseq;
  size_t kc, vc, hs, hmid, xa, xb, xc, pa, pc, xs, qkv, apart, aout, pgpart, rstd, act, logits, hpart, rope, target,
      dpg0, dpg1, dpx, dpdec, tok, seqtok, res, dlogits, srec, q8, total;
  int xld, nch_max, nz_max, ntile;
};

bool cfg_valid(const lss_config* c, std::string* why) {
  auto fail = [&](const char* m) { if (why) *why = m; return false; };
  if (!c) return fail("null config");
  if (c->n_layers < 1 || c->d_model < 16 || c->n_heads < 1 || c->n_kv_heads < 1 || c->ffn_dim < 16 ||
      c->vocab < 1)
    return fail("non-positive model dimension");
  if (c->head_dim != 64 && c->head_dim != 128) return fail("head_dim must be 64 or 128");
  if (c->n_heads % c->n_kv_heads) return fail("n_heads must be a multiple of n_kv_heads");
  // whole 4-vector groups of the projection loop: 32 elements (bf16) / 16 (float32)
  const int kq = c->dtype == LSS_BF16 ? 32 : 16;
  if (c->d_model % kq || c->ffn_dim % kq || c->vocab % 16)
    return fail("d_model, ffn_dim must be multiples of 32 (bf16) / 16 (float32), vocab of 16");
  if (c->d_model > 8192) return fail("d_model > 8192");
  // projection depth of the decode GEMV: GV_WAVES waves x 8 chunks of 64 lanes x 16 bytes
  const long kmax = (long)GV_WAVES * 8 * gv_chunk(c->dtype == LSS_BF16 ? 2 : 4);
  if (c->ffn_dim > kmax || (long)c->n_heads * c->head_dim > kmax)
    return fail("ffn_dim and n_heads * head_dim must be <= 32768 (bf16) / 16384 (float32)");
  if (c->dtype != LSS_F32 && c->dtype != LSS_BF16) return fail("dtype must be LSS_F32 or LSS_BF16");
  if (c->kv_dtype != LSS_F32 && c->kv_dtype != LSS_BF16) return fail("kv_dtype must be LSS_F32 or LSS_BF16");
  if (c->max_rows < 1 || c->max_rows > LSS_ROWS_MAX) return fail("max_rows out of [1, 64]");
  if (c->max_seq < 2 || c->max_seq > 4096) return fail("max_seq out of [2, 4096]");
  if (c->max_seqs < 0 || c->max_seqs > LSS_SEQS_MAX) return fail("max_seqs out of [0, 64]");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return fail("bad rms_eps / rope_theta");
  return true;
}

Layout make_layout(const lss_config* c) {
  Layout L{};
  const size_t elt = c->kv_dtype == LSS_BF16 ? 2 : 4;
  const size_t R = c->max_rows, d = c->d_model, F = c->ffn_dim, hd = c->head_dim;
  const size_t Hq = c->n_heads, Hkv = c->n_kv_heads, V = c->vocab, NL = c->n_layers;
  const size_t S = (size_t)std::max(1, c->max_seqs);
  L.nseq = (int)S;
  L.xld = (int)std::max({d, F, Hq * hd});
  L.nch_max = (c->max_seq + ATT_CH - 1) / ATT_CH;
  // query blocks of a pass: a batched pass rounds up per sequence
  L.nz_max = (int)(((Hq / Hkv) * R + ATT_QB - 1) / ATT_QB) + (S > 1 ? (int)std::min<size_t>(S, ATT_SEQ_MAX) : 0);
  L.ntile = (int)((V + 15) / 16);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  L.seq_kv = NL * Hkv * (size_t)c->max_seq * hd * elt;
  L.kc = take(S * L.seq_kv);
  L.vc = take(S * L.seq_kv);
  L.hs = take((NL + 1) * R * d * 4);
  L.hmid = take(R * d * 4);
  // projection inputs (4 bytes per element in both formats) and partial sums of squares
  L.xa = take(R * d * 4);
  L.xb = take(R * (size_t)std::max(F, Hq * hd) * 4);
  L.xc = take(R * d * 4);
  L.pa = take(R * (d / 16) * 4);
  L.pc = take(R * (d / 16) * 4);
  L.xs = take(R * 4);
  L.qkv = take(R * (Hq + 2 * Hkv) * hd * 4);
  L.apart = take(Hkv * (size_t)L.nz_max * L.nch_max * ATT_QB * (hd + 2) * 4);
  L.aout = take(R * Hq * hd * 4);
  {  // split partials of the prefill / layer-selection GEMM: max over the projections of S x NACC x N
    const int wb = c->dtype == LSS_BF16 ? 2 : 4;
    const size_t qn = (Hq + 2 * Hkv) * hd;
    const size_t a = pg_splits((int)qn, (int)d, wb) * qn, b = pg_splits((int)d, (int)(Hq * hd), wb) * d,
                 g = 2 * pg_splits((int)F, (int)d, wb) * F, dn = pg_splits((int)d, (int)F, wb) * d;
    L.pgpart = take(std::max({a, b, g, dn}) * R * 4);
  }
  L.rstd = take(R * 4);
  L.act = take(R * F * 4);
  L.logits = take(R * V * 4);
  L.hpart = take(R * (size_t)L.ntile * HEAD_PART * 4);
  L.rope = take((size_t)c->max_seq * (hd / 2) * 8);
  L.target = take(S * (NL + 1) * d * 4);
  L.dpg0 = take(R * d * 4);
  L.dpg1 = take(R * d * 4);
  L.dpx = take(R * d * 4);
  L.dpdec = take((NL + 1) * (NL + 1) * 3 * 4);
  L.tok = take(S * kTokSlots * 4);
  L.seqtok = take((size_t)c->max_seq * 4);
  L.res = take((S + 1) * sizeof(HeadRes));        // one per sequence, then the batched passes' rows
  L.dlogits = take((size_t)std::min<size_t>(kWinMax, R) * V * 4);       // sampling: draft logits per window slot
  L.srec = take((size_t)((V + SPEC_RES_PER_WG - 1) / SPEC_RES_PER_WG) * 4 * 4);
  L.q8 = take(R * (size_t)L.xld);                  // int8-weight draft: activation codes
  L.total = off;
  return L;
}

struct LayerW {
  const float* attn_norm;
  const void *wq, *wk, *wv, *wo;
  const float* ffn_norm;
  const void *wg, *wu, *wd;
};

// int8 copy of one layer's projections (codes [N][K], row scales [N]) in
// the order q, k, v, o, gate, up, down
struct LayerW8 {
  const int8_t* q[7];
  const float* s[7];
};

// (rows, columns) of the seven projections of a layer
void w8_shapes(const lss_config* c, int (&n)[7], int (&k)[7]) {
  const int d = c->d_model, F = c->ffn_dim, qd = c->n_heads * c->head_dim, kvd = c->n_kv_heads * c->head_dim;
  const int nn[7] = {qd, kvd, kvd, d, F, F, d}, kk[7] = {d, d, d, qd, d, d, F};
  for (int i = 0; i < 7; ++i) { n[i] = nn[i]; k[i] = kk[i]; }
}
// bytes of the int8 copy of every layer; offsets[l][i] of codes and scales
size_t w8_layout(const lss_config* c, std::vector<std::array<size_t, 14>>* offs) {
  int n[7], k[7];
  w8_shapes(c, n, k);
  size_t off = 0;
  if (offs) offs->resize(c->n_layers);
  for (int l = 0; l < c->n_layers; ++l)
    for (int i = 0; i < 7; ++i) {
      if (offs) (*offs)[l][i] = off;
      off += align_up((size_t)n[i] * k[i]);
      if (offs) (*offs)[l][7 + i] = off;
      off += align_up((size_t)n[i] * 4);
    }
  return off;
}

// MODE_TREE: a tree verify pass; MODE_TREE_DRAFT: a tree draft step (rows =
// the nodes of one depth of consecutive branches)
// MODE_BATCH / MODE_BATCH_DRAFT: the rows of a batched pass (verify rows,
// draft rows) of the sequences in lss_engine::pass
enum RowMode { MODE_CAUSAL = 0, MODE_DRAFT = 1, MODE_DP = 2, MODE_TREE = 3, MODE_TREE_DRAFT = 4, MODE_BATCH = 5,
               MODE_BATCH_DRAFT = 6 };

}  // namespace

// state of one sequence while it is not the current one (lss_seq_select);
// the current sequence's state lives in the engine's own fields
struct SeqState {
  int p = 0, win = 0, tree = 0, tree_D = 1;
  std::vector<uint32_t> valid;
  bool have_seq = false, pending_accept = false;
  int verify_rows = 0;
  bool have_target = false;
  int target_pos = 0;
};

// sequence i of a batched pass: its rows and position (lss_batch_*)
struct PassSeq {
  int seq, row0, M, pos0;
};

// decode-GEMV grid policy of an engine (lss_set_gemv_grid)
#define LSS_GEMV_WGS_PER_CU 1
struct GemvLaunch {
  int ncu = 0, gmax_cu = 0;   // compute units; workgroups per unit (0: one per tile)
};

struct lss_engine {
  lss_config cfg{};
  Layout lay{};
  hipStream_t stream = nullptr;
  bool bf16 = false;     // weights
  bool kv16 = false;     // KV cache
  const void* embed = nullptr;
  const float* final_norm = nullptr;
  const void* lm_head = nullptr;
  std::vector<LayerW> layers;
  char* ws = nullptr;
  // device buffers
  void *kc = nullptr, *vc = nullptr;
  float *hs, *hmid, *xs, *qkv, *apart, *aout, *act, *logits, *hpart, *target, *dpg[2], *dpx, *dpdec;
  float *pgpart, *rstd;
  float *dlogits = nullptr, *srec = nullptr;  // sampling: draft logits of the window slots, replacement-draw records
  int8_t* q8 = nullptr;                       // int8-weight draft: activation codes of the row
  int tree = 0;                               // width of the pending tree window (0: a chain)
  int tree_D = 1;                             // its depth
  int tree_step = 0, tree_b0 = 0;             // MODE_TREE_DRAFT rows: depth, branch of the first row
  std::vector<LayerW8> w8;                    // int8 weight copies (lss_attach_w8), empty until attached
  void *xa, *xb, *xc;   // projection inputs: layer input (attention-norm gain), attention / FFN output, mid-layer
  float *pa, *pc;       // partial sums of squares of the residual rows behind xa and xc
  float2* rope;
  int32_t *tok, *seqtok;
  HeadRes* res;
  // pinned host mirrors
  HeadRes* hres = nullptr;
  int32_t* hstage = nullptr;
  // sequences: the current one (its state in the fields below), the saved
  // state of every sequence, and the per-sequence blocks of the workspace
  int nseq = 1, cur = 0;
  std::vector<SeqState> seqs;
  char *kc_all = nullptr, *vc_all = nullptr;
  int32_t* tok_all = nullptr;
  float* target_all = nullptr;
  HeadRes *res_all = nullptr, *hres_all = nullptr;   // device / pinned host, nseq + 1 (the last: batched rows)
  std::vector<PassSeq> pass;                         // sequences of the running batched pass
  // sequence state
  int p = 0;                  // committed length
  int win = 0;                // drafted tokens in the window
  std::vector<uint32_t> valid;  // per layer: window slots whose KV this layer wrote
  bool have_seq = false;
  bool pending_accept = false;
  int verify_rows = 0;
  int logits_rows = 0;
  bool have_target = false;
  int target_pos = 0;
  // speculative sampling (lss_set_sampling): 1 / temperature (0: greedy) and seed
  float inv_t = 0.f;
  uint64_t seed = 0;
  // projections of draft / verify rows go through the vector-ALU GEMV
  // (one arithmetic for every row count); prefill and layer selection
  // through the MFMA kernels
  bool gemv = false;
  GemvLaunch gvl;
  // decode rows of bf16 weights (lss_set_decode_kernel): MFMA GEMM (one
  // launch for up to 16 rows) or the vector-ALU GEMV, separately for the
  // full-model rows (verify, greedy steps) and the draft rows
  bool decode_mfma = false, draft_mfma = false;
  bool in_draft = false;       // a draft step is running
  // kernel timing (lss_profile_kernel)
  int prof_epi = -1, prof_rows = 0;
  std::vector<hipEvent_t> ev_start, ev_stop;
  int ev_used = 0;
  double prof_ms = 0.0;
  int64_t prof_launches = 0, prof_bytes = 0;
  std::string err;
};

namespace {

int fail(lss_engine* e, int code, const std::string& msg) {
  if (e) e->err = msg;
  return code;
}

#define HIPCHK(expr)                                                                    \
  do {                                                                                  \
    hipError_t _s = (expr);                                                             \
    if (_s != hipSuccess)                                                               \
      return fail(e, LSS_EHIP, std::string(#expr) + ": " + hipGetErrorString(_s));     \
  } while (0)

int check_launch(lss_engine* e, const char* what) {
  hipError_t s = hipGetLastError();
  if (s != hipSuccess) return fail(e, LSS_EHIP, std::string(what) + ": " + hipGetErrorString(s));
  return LSS_OK;
}

size_t kv_layer_elems(const lss_engine* e) {
  return (size_t)e->cfg.n_kv_heads * e->cfg.max_seq * e->cfg.head_dim;
}
void* kc_layer(lss_engine* e, int l) {
  const size_t elt = e->kv16 ? 2 : 4;
  return (char*)e->kc + (size_t)l * kv_layer_elems(e) * elt;
}
void* vc_layer(lss_engine* e, int l) {
  const size_t elt = e->kv16 ? 2 : 4;
  return (char*)e->vc + (size_t)l * kv_layer_elems(e) * elt;
}
float* hs_row(lss_engine* e, int l, int m) {
  return e->hs + ((size_t)l * e->cfg.max_rows + m) * e->cfg.d_model;
}

// the current sequence's fields to its saved state, and back
void seq_save(lss_engine* e) {
  SeqState& q = e->seqs[e->cur];
  q.p = e->p; q.win = e->win; q.tree = e->tree; q.tree_D = e->tree_D;
  q.valid = e->valid;
  q.have_seq = e->have_seq; q.pending_accept = e->pending_accept;
  q.verify_rows = e->verify_rows;
  q.have_target = e->have_target; q.target_pos = e->target_pos;
}
void seq_load(lss_engine* e, int i) {
  const SeqState& q = e->seqs[i];
  e->cur = i;
  e->p = q.p; e->win = q.win; e->tree = q.tree; e->tree_D = q.tree_D;
  e->valid = q.valid;
  e->have_seq = q.have_seq; e->pending_accept = q.pending_accept;
  e->verify_rows = q.verify_rows;
  e->have_target = q.have_target; e->target_pos = q.target_pos;
  e->kc = e->kc_all + (size_t)i * e->lay.seq_kv;
  e->vc = e->vc_all + (size_t)i * e->lay.seq_kv;
  e->tok = e->tok_all + (size_t)i * kTokSlots;
  e->target = e->target_all + (size_t)i * (e->cfg.n_layers + 1) * e->cfg.d_model;
  e->res = e->res_all + i;
  e->hres = e->hres_all + i;
}

// ------------------------------------------------------------------ launches
// Launch one projection kernel.  With t0/t1 set the launch goes through
// hipExtLaunchKernelGGL, which stamps the two events from the kernel's own
// dispatch (start and end of execution), not from separate marker packets.
template <typename K>
void launch_k(K kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, hipEvent_t t0, hipEvent_t t1,
              const GemmArgs& ga) {
  if (t0) hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, s, t0, t1, 0u, ga);
  else hipLaunchKernelGGL(kern, grid, block, lds, s, ga);
}


// GemmArgs of rows r0 .. r0 + Mg - 1 of a projection
GemmArgs rows_from(const GemmArgs& ga, int r0, int Mg) {
  GemmArgs g = ga;
  g.M = Mg;
  g.A = (const char*)ga.A + (size_t)r0 * ga.lda * 4;
  if (ga.pin) g.pin = ga.pin + (size_t)r0 * (ga.K / 16);
  if (ga.xs) g.xs = ga.xs + r0;
  if (ga.Y) g.Y = ga.Y + (size_t)r0 * ga.ldy;
  if (ga.R) g.R = ga.R + (size_t)r0 * ga.ldr;
  if (ga.xo) g.xo = (char*)ga.xo + (size_t)r0 * ga.ldo * 4;
  if (ga.po) g.po = ga.po + (size_t)r0 * (ga.N / 16);
  if (ga.part) g.part = ga.part + (size_t)r0 * (ga.N / 16) * HEAD_PART;
  g.pos0 = ga.pos0 + r0 * ga.pos_step;
  return g;
}

// chunks per wave a vector-GEMV launch over K needs (a power of two)
int gemv_ncw(int K, int wbytes) {
  const int CH = gv_chunk(wbytes);
  const int per = ((K + CH - 1) / CH + GV_WAVES - 1) / GV_WAVES;
  int ncw = 1;
  while (ncw < per) ncw *= 2;
  return ncw;
}
// rows per vector-GEMV launch: the activation chunks of a wave stay in
// registers (MB x NCW <= GV_ACT_MAX; 8 rows only with one chunk per wave,
// where the accumulators still fit without spilling)
int gemv_cap(int K, int wbytes) {
  const int ncw = gemv_ncw(K, wbytes);
  return ncw == 1 ? GV_MB_MAX : std::max(1, std::min(4, GV_ACT_MAX / ncw));
}

// 8-row tiles for gate/up and for one-row q/k/v launches (more workgroups);
// 16-row tiles otherwise (multi-row q/k/v measured faster with them).  The
// tile size does not change any output bit.
template <int EPI, int MB> constexpr int gemv_tile() {
  return (EPI == EPI_SWIGLU || (EPI == EPI_STORE && MB == 1)) ? 8 : 16;
}

// Workgroups of one decode-GEMV launch.  gmax_cu = 0: one per tile.
// Otherwise, with at most gmax = gmax_cu workgroups per compute unit (capped
// by the kernel's occupancy): launches of at most 4 gmax tiles keep one
// workgroup per tile (several resident workgroups per compute unit fill it
// faster than a short walk); larger ones take
// ceil(tiles / ceil(tiles / gmax)) workgroups, each walking the same number
// of tiles give or take one.
int gemv_grid(int ntile, int ncu, int gmax_cu, int occ) {
  if (gmax_cu <= 0 || ncu <= 0) return ntile;
  const int gmax = ncu * std::max(1, std::min(gmax_cu, occ));
  if (ntile <= 4 * gmax) return ntile;
  const int per = (ntile + gmax - 1) / gmax;
  return (ntile + per - 1) / per;
}

template <typename WT, int MB, int NCW, int EPI>
void gemv_go(const GemmArgs& g, const GemvLaunch& gl, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  constexpr int TR = gemv_tile<EPI, MB>();
  static const int occ = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_gemv<WT, MB, NCW, EPI, TR>, 64 * GV_WAVES, 0) !=
            hipSuccess || nb < 1)
      nb = 1;
    return nb;
  }();
  const int ntile = (g.N + TR - 1) / TR;
  const dim3 grid(gemv_grid(ntile, gl.ncu, gl.gmax_cu, occ)), block(64 * GV_WAVES);
  launch_k(k_gemv<WT, MB, NCW, EPI, TR>, grid, block, 0, s, t0, t1, g);
}

template <typename WT, int EPI, int NCW>
void gemv_launch(const GemmArgs& g, const GemvLaunch& gl, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if constexpr (NCW == 1) {
    if (g.M == 1) gemv_go<WT, 1, 1, EPI>(g, gl, s, t0, t1);
    else if (g.M == 2) gemv_go<WT, 2, 1, EPI>(g, gl, s, t0, t1);
    else if (g.M <= 4) gemv_go<WT, 4, 1, EPI>(g, gl, s, t0, t1);
    else gemv_go<WT, 8, 1, EPI>(g, gl, s, t0, t1);
  } else if constexpr (NCW == 2 || NCW == 4) {
    if (g.M == 1) gemv_go<WT, 1, NCW, EPI>(g, gl, s, t0, t1);
    else if (g.M == 2) gemv_go<WT, 2, NCW, EPI>(g, gl, s, t0, t1);
    else gemv_go<WT, 4, NCW, EPI>(g, gl, s, t0, t1);
  } else {
    if (g.M == 1) gemv_go<WT, 1, 8, EPI>(g, gl, s, t0, t1);
    else gemv_go<WT, 2, 8, EPI>(g, gl, s, t0, t1);
  }
}

// M rows in launches of at most gemv_cap rows (each row's arithmetic is the
// same in any launch)
template <typename WT, int EPI>
void gemv_mt(const GemmArgs& ga, const GemvLaunch& gl, hipStream_t s, hipEvent_t t0 = nullptr,
             hipEvent_t t1 = nullptr) {
  const int ncw = gemv_ncw(ga.K, sizeof(WT));
  const int cap = gemv_cap(ga.K, sizeof(WT));
  for (int r0 = 0; r0 < ga.M; r0 += cap) {
    const int Mg = std::min(cap, ga.M - r0);
    const GemmArgs g = (r0 == 0 && Mg == ga.M) ? ga : rows_from(ga, r0, Mg);
    if (ncw == 1) gemv_launch<WT, EPI, 1>(g, gl, s, t0, t1);
    else if (ncw == 2) gemv_launch<WT, EPI, 2>(g, gl, s, t0, t1);
    else if (ncw == 4) gemv_launch<WT, EPI, 4>(g, gl, s, t0, t1);
    else gemv_launch<WT, EPI, 8>(g, gl, s, t0, t1);
  }
}

// MFMA decode GEMM: one launch for all M <= 16 rows, tiles of 16 or 32
// weight rows and 4 or 8 MFMA waves per workgroup by the rules below.  The
// tile width changes no output bit; the wave count fixes the split of K and
// is a function of the projection alone.
#ifndef VG_ST
#define VG_ST 2
#endif
template <int EPI, int TN, int W>
void vgemm_go(const GemmArgs& g, const GemvLaunch& gl, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  static const int occ = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_vgemm<EPI, TN, VG_ST, W>, 64 * (W + 1), 0) !=
            hipSuccess || nb < 1)
      nb = 1;
    return nb;
  }();
  // policy > 0: no more workgroups than are resident at once, each walking
  // an equal share of the tiles (give or take one)
  const int ntile = (g.N + TN - 1) / TN;
  int nwg = ntile;
  if (gl.gmax_cu > 0 && gl.ncu > 0 && ntile > gl.ncu * occ) {
    const int per = (ntile + gl.ncu * occ - 1) / (gl.ncu * occ);
    nwg = (ntile + per - 1) / per;
  }
  const dim3 grid(nwg), block(64 * (W + 1));
  launch_k(k_vgemm<EPI, TN, VG_ST, W>, grid, block, 0, s, t0, t1, g);
}
// Tiles of 32 weight rows halve the activation loads per weight byte of
// 16-row tiles but halve the workgroups.  Measured (one row / nine rows,
// HIP events, interleaved A/B): 32-row tiles win where they give 0.75 to 1
// tile per compute unit (q/k/v at 8B, 192 tiles: 13.2 against 15.9 us;
// the 8192-row projections at 70B, 256 tiles: 51.6 against 54.8 us) and
// for the LM head's thousands of tiles; 16-row tiles win below (the 4096-row
// projections at 8B, 128 tiles) and above (q/k/v at 70B, 320 tiles: 39.2
// against 44.6 us), where the extra workgroups keep more loads in flight.
// gate/up holds two matrices per tile and always takes 16 rows.
//
// MFMA waves per workgroup: 8 for the q/k/v and gate/up projections of depth
// K >= 8192 (70B: q/k/v 39.2 -> 35.3 us at one row, gate/up 151.7 -> 144.8
// at one row and 166.2 -> 151.8 at nine), 4 otherwise (at K = 4096 every
// projection, and at 70B the LM head, measured slower with 8).  The choice
// depends on the projection only, never on the row count.
template <int EPI>
void vgemm(const GemmArgs& g, const GemvLaunch& gl, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const bool w8 = g.K >= 8192 && (EPI == EPI_STORE || EPI == EPI_SWIGLU);
  if constexpr (EPI != EPI_SWIGLU) {
    const long t32 = g.N / 32, ncu = gl.ncu;
    if (ncu > 0 && ((4 * t32 >= 3 * ncu && t32 <= ncu) || t32 >= 4 * ncu)) {
      if (w8) vgemm_go<EPI, 32, 8>(g, gl, s, t0, t1);
      else vgemm_go<EPI, 32, 4>(g, gl, s, t0, t1);
      return;
    }
  }
  if (w8) vgemm_go<EPI, 16, 8>(g, gl, s, t0, t1);
  else vgemm_go<EPI, 16, 4>(g, gl, s, t0, t1);
}

// Prefill / layer-selection projection: 1/rms rows, split MFMA GEMM, split
// sum + epilogue.  The timing events (if any) bracket the GEMM launch.
template <typename WT, int EPI>
void pgemm(lss_engine* e, const GemmArgs& ga, hipEvent_t t0, hipEvent_t t1) {
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  PgArgs pa{};
  for (int i = 0; i < 3; ++i) { pa.w[i] = ga.w[i]; pa.nseg[i] = ga.nseg[i]; }
  pa.w2 = ga.w2; pa.N = ga.N; pa.K = ga.K; pa.A = ga.A; pa.lda = ga.lda; pa.M = ga.M;
  pa.S = pg_splits(ga.N, ga.K, sizeof(WT));
  pa.part = e->pgpart;
  hipStream_t s = e->stream;
  if (ga.scale == SCALE_NORM)
    hipLaunchKernelGGL(k_rstd, dim3(ga.M), dim3(256), 0, s, ga.pin, ga.K / 16, ga.K, ga.eps, e->rstd);
  const dim3 grid((ga.N + PG_TN - 1) / PG_TN, pa.S), block(256);
  auto go = [&](auto kern) {
    if (t0) hipExtLaunchKernelGGL(kern, grid, block, 0u, s, t0, t1, 0u, pa);
    else hipLaunchKernelGGL(kern, grid, block, 0, s, pa);
  };
  switch ((ga.M + 15) / 16) {
    case 1: go(k_pgemm<WT, 1, NACC>); break;
    case 2: go(k_pgemm<WT, 2, NACC>); break;
    case 3: go(k_pgemm<WT, 3, NACC>); break;
    default: go(k_pgemm<WT, 4, NACC>); break;
  }
  hipLaunchKernelGGL((k_pepi<WT, EPI>), dim3((ga.N + 15) / 16), dim3(256), 0, s, ga, (const float*)e->pgpart, pa.S,
                     (const float*)e->rstd);
}

// Sum the elapsed times of recorded event pairs (the stream must be synced).
void prof_resolve(lss_engine* e) {
  for (int i = 0; i < e->ev_used; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e->ev_start[i], e->ev_stop[i]) == hipSuccess) e->prof_ms += ms;
  }
  e->ev_used = 0;
}

template <int EPI>
void gemm(lss_engine* e, const GemmArgs& ga) {
  // draft / verify rows, and any launch of at most 16 (MFMA decode GEMM) or
  // 8 (vector GEMV) rows, take the decode kernel; with the MFMA kernel more
  // than 16 rows go in 16-row launches (never to another kernel, whose
  // arithmetic would differ from the greedy rows')
  const bool mf = e->bf16 && (e->in_draft ? e->draft_mfma : e->decode_mfma);
  const bool vec = e->gemv || ga.M <= (mf ? VG_MMAX : 8);
  const bool one_launch = !vec || (mf && ga.M <= VG_MMAX) || ga.M <= gemv_cap(ga.K, e->bf16 ? 2 : 4);
  const bool prof = e->prof_epi == EPI && (e->prof_rows == 0 || e->prof_rows == ga.M) && one_launch;
  if (prof) {
    if (e->ev_used == (int)e->ev_start.size()) {
      (void)hipStreamSynchronize(e->stream);
      prof_resolve(e);
    }
  }
  hipEvent_t t0 = prof ? e->ev_start[e->ev_used] : nullptr, t1 = prof ? e->ev_stop[e->ev_used] : nullptr;
  if (vec) {
    if (mf) {                                      // blocks of 16 rows, each row's arithmetic unchanged
      for (int r0 = 0; r0 < ga.M; r0 += VG_MMAX)
        vgemm<EPI>(ga.M <= VG_MMAX ? ga : rows_from(ga, r0, std::min(VG_MMAX, ga.M - r0)), e->gvl, e->stream, t0, t1);
    } else if (e->bf16) gemv_mt<uint16_t, EPI>(ga, e->gvl, e->stream, t0, t1);
    else gemv_mt<float, EPI>(ga, e->gvl, e->stream, t0, t1);
  } else {
    if (e->bf16) pgemm<uint16_t, EPI>(e, ga, t0, t1);
    else pgemm<float, EPI>(e, ga, t0, t1);
  }
  if (prof) {
    e->ev_used++;
    const int64_t elt = e->bf16 ? 2 : 4;
    const int64_t nw = (EPI == EPI_SWIGLU) ? 2 : 1;
    e->prof_launches++;
    // weights + activation rows read (4 bytes per element) + rows written (float32 and/or projection input)
    const int64_t outw = (ga.Y && !(EPI == EPI_SWIGLU && ga.xo) ? 4 : 0) + (ga.xo ? 4 : 0);
    e->prof_bytes += nw * (int64_t)ga.N * ga.K * elt + (int64_t)ga.M * ga.K * 4 + (int64_t)ga.M * ga.N * outw +
                     (EPI == EPI_RESID ? (int64_t)ga.M * ga.N * 4 : 0);
  }
}

GemmArgs gemm_args(const void* w, int N, int K, const void* A, int lda, int M, float* Y, int ldy) {
  GemmArgs ga{};
  ga.w[0] = w; ga.w[1] = w; ga.w[2] = w;
  ga.nseg[0] = N; ga.nseg[1] = 0; ga.nseg[2] = 0;
  ga.N = N; ga.K = K; ga.A = A; ga.lda = lda; ga.M = M; ga.Y = Y; ga.ldy = ldy;
  ga.scale = SCALE_NONE;
  return ga;
}

// projection-format row offset (both formats take 4 bytes per element)
const void* xrow(const void* x, int ld, int m) { return (const char*)x + (size_t)m * ld * 4; }

template <typename KT, typename WT>
void attention(lss_engine* e, int l, int M, int mode, int pos0, int quant) {
  const auto& c = e->cfg;
  const int hd = c.head_dim;
  AttnArgs a{};
  a.qkv = e->qkv; a.ldqkv = (c.n_heads + 2 * c.n_kv_heads) * hd;
  a.cs = e->rope;
  a.kc = kc_layer(e, l); a.vc = vc_layer(e, l);
  a.max_seq = c.max_seq; a.Hq = c.n_heads; a.Hkv = c.n_kv_heads; a.M = M;
  a.pos0 = pos0; a.pos_step = mode == MODE_DP ? 0 : 1;
  const bool tree = mode == MODE_TREE || mode == MODE_TREE_DRAFT;
  a.tree = tree ? 1 : 0;
  a.tree_D = e->tree_D;
  a.tree_step = mode == MODE_TREE_DRAFT ? e->tree_step : 0;
  a.tree_b0 = mode == MODE_TREE_DRAFT ? e->tree_b0 : 0;
  a.part = e->apart; a.nz_max = e->lay.nz_max; a.nch_max = e->lay.nch_max;
  a.out = e->aout;
  a.xo = quant ? nullptr : e->xb;
  a.scale = (float)(1.0 / std::sqrt((double)hd));
  int kmax;
  if (mode == MODE_CAUSAL) { a.lim_base = pos0 + 1; a.lim_step = 1; a.wbase = 0; a.wmask = 0; kmax = pos0 + M; }
  else if (mode == MODE_TREE) { a.lim_base = pos0 + 1; a.lim_step = 0; a.wbase = 0; a.wmask = 0; kmax = pos0 + M; }
  else if (mode == MODE_TREE_DRAFT) {             // last row's slot: pos0 + j + (b0 + M - 1) D
    a.lim_base = pos0; a.lim_step = 0; a.wbase = pos0; a.wmask = e->valid[l];   // p + i by valid bit i
    kmax = pos0 + e->tree_step + (e->tree_b0 + M - 1) * e->tree_D + 1;
  }
  else if (mode == MODE_DRAFT) { a.lim_base = e->p; a.lim_step = 0; a.wbase = e->p; a.wmask = e->valid[l]; kmax = pos0 + 1; }
  else { a.lim_base = pos0; a.lim_step = 0; a.wbase = 0; a.wmask = 0; a.self_kv = 1; kmax = pos0; }
  a.nch = std::max(1, (kmax + ATT_CH - 1) / ATT_CH);
  const int G = c.n_heads / c.n_kv_heads;
  a.nz = (G * M + ATT_QB - 1) / ATT_QB;
  const int mq = std::min(ATT_QB, G * M);             // merge workgroups per query block and kv head
  const dim3 grid(a.nch, c.n_kv_heads, a.nz);
  if (hd == 128) {
    if (tree) hipLaunchKernelGGL((k_attention<KT, WT, 128, true>), grid, dim3(ATT_THREADS), 0, e->stream, a);
    else hipLaunchKernelGGL((k_attention<KT, WT, 128>), grid, dim3(ATT_THREADS), 0, e->stream, a);
    hipLaunchKernelGGL((k_attn_merge<WT, 128>), dim3(mq, c.n_kv_heads, a.nz), dim3(128), 0, e->stream, a);
  } else {
    if (tree) hipLaunchKernelGGL((k_attention<KT, WT, 64, true>), grid, dim3(ATT_THREADS), 0, e->stream, a);
    else hipLaunchKernelGGL((k_attention<KT, WT, 64>), grid, dim3(ATT_THREADS), 0, e->stream, a);
    hipLaunchKernelGGL((k_attn_merge<WT, 64>), dim3(mq, c.n_kv_heads, a.nz), dim3(64), 0, e->stream, a);
  }
}

// attention of a batched pass: every sequence of e->pass with its own rows,
// cache block, position and visibility (verify rows causal from its
// committed length; a draft row sees its prefix and its window slots that
// this layer wrote), in one launch pair
template <typename KT, typename WT>
void attention_batch(lss_engine* e, int l, int mode, int quant) {
  const auto& c = e->cfg;
  const int hd = c.head_dim;
  const bool draft = mode == MODE_BATCH_DRAFT;
  AttnArgs a{};
  a.qkv = e->qkv; a.ldqkv = (c.n_heads + 2 * c.n_kv_heads) * hd;
  a.cs = e->rope;
  const size_t elt = e->kv16 ? 2 : 4;
  a.kc = e->kc_all + (size_t)l * kv_layer_elems(e) * elt;
  a.vc = e->vc_all + (size_t)l * kv_layer_elems(e) * elt;
  a.seq_stride = (int64_t)e->lay.seq_kv;
  a.max_seq = c.max_seq; a.Hq = c.n_heads; a.Hkv = c.n_kv_heads;
  a.pos_step = 1;
  a.lim_step = draft ? 0 : 1;
  a.part = e->apart; a.nz_max = e->lay.nz_max; a.nch_max = e->lay.nch_max;
  a.out = e->aout;
  a.xo = quant ? nullptr : e->xb;
  a.scale = (float)(1.0 / std::sqrt((double)hd));
  const int G = c.n_heads / c.n_kv_heads;
  AttnSeqs q{};
  q.n = (int)e->pass.size();
  int nch = 1, mmax = 1, rows = 0;
  q.zs[0] = 0;
  for (int i = 0; i < q.n; ++i) {
    const PassSeq& ps = e->pass[i];
    const SeqState& st = e->seqs[ps.seq];
    q.row0[i] = ps.row0; q.M[i] = ps.M; q.pos0[i] = ps.pos0; q.slot[i] = ps.seq;
    int kmax;
    if (draft) {
      q.lim_base[i] = st.p; q.wbase[i] = st.p; q.wmask[i] = st.valid[l];
      kmax = ps.pos0 + 1;
    } else {
      q.lim_base[i] = ps.pos0 + 1; q.wbase[i] = 0; q.wmask[i] = 0;
      kmax = ps.pos0 + ps.M;
    }
    q.nch[i] = std::max(1, (kmax + ATT_CH - 1) / ATT_CH);
    q.zs[i + 1] = q.zs[i] + (G * ps.M + ATT_QB - 1) / ATT_QB;
    nch = std::max(nch, q.nch[i]);
    mmax = std::max(mmax, ps.M);
    rows += ps.M;
  }
  a.M = rows;
  a.nch = nch;
  a.nz = q.zs[q.n];
  const int mq = std::min(ATT_QB, G * mmax);
  const dim3 grid(nch, c.n_kv_heads, a.nz);
  if (hd == 128) {
    hipLaunchKernelGGL((k_attention_b<KT, WT, 128>), grid, dim3(ATT_THREADS), 0, e->stream, a, q);
    hipLaunchKernelGGL((k_attn_merge_b<WT, 128>), dim3(mq, c.n_kv_heads, a.nz), dim3(128), 0, e->stream, a, q);
  } else {
    hipLaunchKernelGGL((k_attention_b<KT, WT, 64>), grid, dim3(ATT_THREADS), 0, e->stream, a, q);
    hipLaunchKernelGGL((k_attn_merge_b<WT, 64>), dim3(mq, c.n_kv_heads, a.nz), dim3(64), 0, e->stream, a, q);
  }
}

template <typename WT>
void attention_w(lss_engine* e, int l, int M, int mode, int pos0, int quant) {
  if (mode == MODE_BATCH || mode == MODE_BATCH_DRAFT) {
    if (e->kv16) attention_batch<uint16_t, WT>(e, l, mode, quant);
    else attention_batch<float, WT>(e, l, mode, quant);
    return;
  }
  if (e->kv16) attention<uint16_t, WT>(e, l, M, mode, pos0, quant);
  else attention<float, WT>(e, l, M, mode, pos0, quant);
}

// RMSNorm + int8 codes of M rows of h into the projection input x (quantized drafts)
// int8 codes of the normalized rows: in the projection format (x), or raw
// into q8 when q8 != nullptr (the int8-weight draft)
void norm_quant(lss_engine* e, const float* h, int M, const float* g, void* x, int8_t* q8 = nullptr) {
  const auto& c = e->cfg;
  if (e->bf16)
    hipLaunchKernelGGL(k_rmsnorm_quant<uint16_t>, dim3(M), dim3(LSS_NORM_THREADS), 0, e->stream, h, c.d_model, g,
                       c.d_model, c.rms_eps, x, e->xs, q8);
  else
    hipLaunchKernelGGL(k_rmsnorm_quant<float>, dim3(M), dim3(LSS_NORM_THREADS), 0, e->stream, h, c.d_model, g,
                       c.d_model, c.rms_eps, x, e->xs, q8);
}

void quant_rows(lss_engine* e, const float* x, int M, int n, void* xo, int8_t* q8 = nullptr) {
  if (e->bf16)
    hipLaunchKernelGGL(k_quant_rows<uint16_t>, dim3(M), dim3(256), 0, e->stream, x, n, n, xo, e->xs, q8);
  else
    hipLaunchKernelGGL(k_quant_rows<float>, dim3(M), dim3(256), 0, e->stream, x, n, n, xo, e->xs, q8);
}

// int8 GEMV of the row e->q8 (scale e->xs[0]) against int8 weights; the
// timing events of lss_profile_kernel bracket it like the bf16 launches
template <int EPI>
void gemm8(lss_engine* e, const GemmArgs& ga) {
  const bool prof = e->prof_epi == EPI + 16 && (e->prof_rows == 0 || e->prof_rows == ga.M);
  if (prof && e->ev_used == (int)e->ev_start.size()) {
    (void)hipStreamSynchronize(e->stream);
    prof_resolve(e);
  }
  hipEvent_t t0 = prof ? e->ev_start[e->ev_used] : nullptr, t1 = prof ? e->ev_stop[e->ev_used] : nullptr;
  const dim3 grid((ga.N + G8_TR - 1) / G8_TR), block(G8_THREADS);
  auto go = [&](auto wt) {
    using WT = decltype(wt);
    const int per = (ga.K + G8_THREADS - 1) / G8_THREADS;
    if (ga.xq || per <= 8) launch_k(k_gemv8<WT, EPI, 8>, grid, block, 0, e->stream, t0, t1, ga);
    else if (per <= 16) launch_k(k_gemv8<WT, EPI, 16>, grid, block, 0, e->stream, t0, t1, ga);
    else if (per <= 32) launch_k(k_gemv8<WT, EPI, 32>, grid, block, 0, e->stream, t0, t1, ga);
    else launch_k(k_gemv8<WT, EPI, 64>, grid, block, 0, e->stream, t0, t1, ga);
  };
  if (e->bf16) go(uint16_t{});
  else go(float{});
  if (prof) {
    e->ev_used++;
    e->prof_launches++;
    const int64_t nw = (EPI == EPI_SWIGLU) ? 2 : 1;
    const int64_t outw = (ga.Y && !(EPI == EPI_SWIGLU && ga.xo) ? 4 : 0) + (ga.xo ? 4 : 0);
    // int8 weights + row scales + activation row (codes, or float32 quantized in place, with the RMSNorm
    // gains and partial sums) + rows written
    e->prof_bytes += nw * ((int64_t)ga.N * ga.K + (int64_t)ga.N * 4) + (int64_t)ga.K * (ga.xq ? 1 : 4) +
                     (ga.scale == SCALE_NORM ? (int64_t)ga.K * 4 + (int64_t)(ga.K / 16) * 4 : 0) +
                     (int64_t)ga.N * outw +
                     (EPI == EPI_RESID ? (int64_t)ga.N * 4 : 0);
  }
}

// projection input + partial sums of squares of M rows of h (row stride d) with gain g
void prep_rows(lss_engine* e, const float* h, int M, const float* g, void* xo, float* po) {
  const int d = e->cfg.d_model;
  if (e->bf16) hipLaunchKernelGGL(k_prep_rows<uint16_t>, dim3(M), dim3(PREP_THREADS), 0, e->stream, h, d, d, g, xo, po);
  else hipLaunchKernelGGL(k_prep_rows<float>, dim3(M), dim3(PREP_THREADS), 0, e->stream, h, d, d, g, xo, po);
}

// One decoder layer on M rows: h_out = layer(h_in).  Rows are consecutive
// positions pos0.. (causal), the single draft slot at pos0, or all at pos0
// (layer selection).  xa_in / pa_in hold h_in's projection input (attention
// norm gain) and its partial sums of squares.  g_next != nullptr: also write
// h_out's projection input with that gain into e->xa / e->pa (rows 0..M-1).
void layer_forward(lss_engine* e, int l, int M, const float* h_in, const void* xa_in, const float* pa_in,
                   float* h_out, const float* g_next, int mode, int pos0, int quant) {
  const auto& c = e->cfg;
  const LayerW& w = e->layers[l];
  const int d = c.d_model, F = c.ffn_dim, hd = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads;
  const int qd = Hq * hd, kvd = Hkv * hd;
  if (quant == 2) {   // int8 weights and int8 activations (one draft row)
    // each int8 GEMV forms its activation codes itself: from the residual row
    // and its partial sums of squares (RMSNorm inputs) or from the float32 row
    const LayerW8& w8 = e->w8[l];
    auto args8 = [&](int i, int N, int K, const float* A, float* Y) {
      GemmArgs ga = gemm_args(w8.q[i], N, K, A, K, M, Y, N);
      ga.wsc[0] = ga.wsc[1] = ga.wsc[2] = w8.s[i];
      return ga;
    };
    {
      GemmArgs ga = args8(0, qd + 2 * kvd, d, h_in, e->qkv);
      ga.scale = SCALE_NORM; ga.pin = pa_in; ga.eps = c.rms_eps; ga.gin = w.attn_norm;
      ga.w[0] = w8.q[0]; ga.nseg[0] = qd; ga.wsc[0] = w8.s[0];
      ga.w[1] = w8.q[1]; ga.nseg[1] = kvd; ga.wsc[1] = w8.s[1];
      ga.w[2] = w8.q[2]; ga.nseg[2] = kvd; ga.wsc[2] = w8.s[2];
      gemm8<EPI_STORE>(e, ga);
    }
    if (e->bf16) attention_w<uint16_t>(e, l, M, mode, pos0, quant);
    else attention_w<float>(e, l, M, mode, pos0, quant);
    {
      GemmArgs ga = args8(3, d, qd, e->aout, e->hmid);
      ga.R = h_in; ga.ldr = d;
      ga.po = e->pc;                                   // partial sums of squares for the FFN norm
      gemm8<EPI_RESID>(e, ga);
    }
    {
      GemmArgs ga = args8(4, F, d, e->hmid, e->act);
      ga.scale = SCALE_NORM; ga.pin = e->pc; ga.eps = c.rms_eps; ga.gin = w.ffn_norm;
      ga.w2 = w8.q[5]; ga.wsc2 = w8.s[5];
      gemm8<EPI_SWIGLU>(e, ga);
    }
    {
      GemmArgs ga = args8(6, d, F, e->act, h_out);
      ga.R = e->hmid; ga.ldr = d;
      if (g_next) { ga.xo = e->xa; ga.ldo = d; ga.go = g_next; ga.po = e->pa; }
      gemm8<EPI_RESID>(e, ga);
    }
    return;
  }
  {
    GemmArgs ga;
    if (quant) {
      norm_quant(e, h_in, M, w.attn_norm, e->xa);
      ga = gemm_args(w.wq, qd + 2 * kvd, d, e->xa, d, M, e->qkv, qd + 2 * kvd);
      ga.scale = SCALE_XS; ga.xs = e->xs;
    } else {
      ga = gemm_args(w.wq, qd + 2 * kvd, d, xa_in, d, M, e->qkv, qd + 2 * kvd);
      ga.scale = SCALE_NORM; ga.pin = pa_in; ga.eps = c.rms_eps;
    }
    ga.w[0] = w.wq; ga.nseg[0] = qd;
    ga.w[1] = w.wk; ga.nseg[1] = kvd;
    ga.w[2] = w.wv; ga.nseg[2] = kvd;
    gemm<EPI_STORE>(e, ga);
  }
  if (e->bf16) attention_w<uint16_t>(e, l, M, mode, pos0, quant);
  else attention_w<float>(e, l, M, mode, pos0, quant);
  if (quant) quant_rows(e, e->aout, M, qd, e->xb);
  {
    GemmArgs ga = gemm_args(w.wo, d, qd, e->xb, qd, M, e->hmid, d);
    if (quant) { ga.scale = SCALE_XS; ga.xs = e->xs; }
    ga.R = h_in; ga.ldr = d;
    if (!quant) { ga.xo = e->xc; ga.ldo = d; ga.go = w.ffn_norm; ga.po = e->pc; }
    gemm<EPI_RESID>(e, ga);
  }
  {
    GemmArgs ga = gemm_args(w.wg, F, d, e->xc, d, M, e->act, F);
    if (quant) {
      norm_quant(e, e->hmid, M, w.ffn_norm, e->xc);
      ga.scale = SCALE_XS; ga.xs = e->xs;
    } else {
      ga.scale = SCALE_NORM; ga.pin = e->pc; ga.eps = c.rms_eps;
      ga.xo = e->xb; ga.ldo = F;
    }
    ga.w2 = w.wu;
    gemm<EPI_SWIGLU>(e, ga);
  }
  if (quant) quant_rows(e, e->act, M, F, e->xb);
  {
    GemmArgs ga = gemm_args(w.wd, d, F, e->xb, F, M, h_out, d);
    if (quant) { ga.scale = SCALE_XS; ga.xs = e->xs; }
    ga.R = e->hmid; ga.ldr = d;
    if (g_next) { ga.xo = e->xa; ga.ldo = d; ga.go = g_next; ga.po = e->pa; }
    gemm<EPI_RESID>(e, ga);
  }
}

// Final norm + LM head on M rows whose projection input (final-norm gain)
// and partial sums of squares start at row r0 of e->xa / e->pa; row m sits
// at position pos0 + m.  Per-row argmax and top-1 probability land in
// res->argmax/pmax[row0 + m].  With sampling on, every row also draws a
// token (the draft stream for a draft row, the full model's otherwise) into
// res->sample[row0 + m] with its log-sum-exp; a draft row keeps its logits
// in the window slot row0 of e->dlogits.
void head(lss_engine* e, int r0, int M, int row0, int pos0, bool draft, HeadRes* res = nullptr) {
  const auto& c = e->cfg;
  const bool samp = e->inv_t > 0.f;
  float* Y = (samp && draft) ? e->dlogits + (size_t)row0 * c.vocab : e->logits;
  GemmArgs ga = gemm_args(e->lm_head, c.vocab, c.d_model, xrow(e->xa, c.d_model, r0), c.d_model, M, Y, c.vocab);
  ga.scale = SCALE_NORM; ga.pin = e->pa + (size_t)r0 * (c.d_model / 16); ga.eps = c.rms_eps;
  ga.part = e->hpart;
  ga.inv_t = e->inv_t; ga.seed = e->seed; ga.purpose = draft ? RNG_DRAFT : RNG_TARGET;
  ga.pos0 = pos0; ga.pos_step = 1;
  gemm<EPI_LOGITS>(e, ga);
  hipLaunchKernelGGL(k_head_reduce, dim3(M), dim3(HEAD_RED_THREADS), 0, e->stream, e->hpart, e->lay.ntile,
                     res ? res : e->res, row0, samp ? 1 : 0, draft ? 1 : 0);
  if (!(samp && draft)) e->logits_rows = M;
}

// embedding rows of tokens tok_dev[0], tok_dev[ts], .. (M rows) into h, with the projection input
// for gain g into e->xa / e->pa
void embed(lss_engine* e, const int32_t* tok_dev, int M, float* h, const float* g, int ts = 1) {
  const auto& c = e->cfg;
  if (e->bf16)
    hipLaunchKernelGGL(k_embed<uint16_t>, dim3(M), dim3(PREP_THREADS), 0, e->stream, (const uint16_t*)e->embed, tok_dev,
                       ts, c.d_model, h, g, e->xa, e->pa);
  else
    hipLaunchKernelGGL(k_embed<float>, dim3(M), dim3(PREP_THREADS), 0, e->stream, (const float*)e->embed, tok_dev,
                       ts, c.d_model, h, g, e->xa, e->pa);
}

// embedding rows of a batched pass: row m's token is e->tok_all[off[m]]
void embed_rows(lss_engine* e, const RowTok& rt, int M, float* h, const float* g) {
  const auto& c = e->cfg;
  if (e->bf16)
    hipLaunchKernelGGL(k_embed_rows<uint16_t>, dim3(M), dim3(PREP_THREADS), 0, e->stream, (const uint16_t*)e->embed,
                       e->tok_all, rt, c.d_model, h, g, e->xa, e->pa);
  else
    hipLaunchKernelGGL(k_embed_rows<float>, dim3(M), dim3(PREP_THREADS), 0, e->stream, (const float*)e->embed,
                       e->tok_all, rt, c.d_model, h, g, e->xa, e->pa);
}

// gain of the RMSNorm that consumes the residual after layer l (l = -1: the
// embedding): the next executed layer's attention norm, else the final norm
const float* next_gain(const lss_engine* e, const uint8_t* mask, int l) {
  for (int j = l + 1; j < e->cfg.n_layers; ++j)
    if (!mask || !mask[j]) return e->layers[j].attn_norm;
  return e->final_norm;
}

// a full-model pass of M causal rows at positions pos0.. whose embeddings are
// tokens tok_dev[0..M): residual stash in hs, projection input of the final
// residual in e->xa (final-norm gain)
void forward_rows(lss_engine* e, const int32_t* tok_dev, int M, int pos0, int mode = MODE_CAUSAL) {
  const int L = e->cfg.n_layers;
  embed(e, tok_dev, M, hs_row(e, 0, 0), next_gain(e, nullptr, -1));
  for (int l = 0; l < L; ++l)
    layer_forward(e, l, M, hs_row(e, l, 0), e->xa, e->pa, hs_row(e, l + 1, 0), next_gain(e, nullptr, l),
                  mode, pos0, 0);
}

int sync_res(lss_engine* e) {
  HIPCHK(hipMemcpyAsync(e->hres, e->res, sizeof(HeadRes), hipMemcpyDeviceToHost, e->stream));
  HIPCHK(hipStreamSynchronize(e->stream));
  if (e->ev_used) prof_resolve(e);
  return LSS_OK;
}

// draft and verify rows: projections through the decode kernels
struct GemvScope {
  lss_engine* e;
  explicit GemvScope(lss_engine* en, bool draft = false) : e(en) {
    e->gemv = true;
    e->in_draft = draft;
  }
  ~GemvScope() {
    e->gemv = false;
    e->in_draft = false;
  }
};

void fill_u32(lss_engine* e, void* p, size_t n, uint32_t v) {
  const size_t blocks = std::min<size_t>((n + 255) / 256, 65536);
  if (n) hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, e->stream, (uint32_t*)p, n, v);
}

// message of the last failed engine creation or stand-alone op on this
// thread (lss_last_error(NULL))
thread_local std::string g_create_err = "no failure";

int create_fail(int code, const std::string& msg) {
  g_create_err = msg;
  return code;
}

// stop tokens of a generation policy: count and ids in range
int check_stop(lss_engine* e, const lss_policy* pol, const char* what) {
  if (pol->n_stop < 0 || pol->n_stop > LSS_STOP_MAX)
    return fail(e, LSS_EINVAL, std::string(what) + ": n_stop must be in [0, LSS_STOP_MAX]");
  for (int i = 0; i < pol->n_stop; ++i)
    if (pol->stop_tokens[i] < 0 || pol->stop_tokens[i] >= e->cfg.vocab)
      return fail(e, LSS_EINVAL, std::string(what) + ": stop token out of range");
  return LSS_OK;
}

bool is_stop(const lss_policy* pol, int32_t tok) {
  for (int i = 0; i < pol->n_stop; ++i)
    if (pol->stop_tokens[i] == tok) return true;
  return false;
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

size_t lss_workspace_bytes(const lss_config* cfg) {
  if (!cfg_valid(cfg, nullptr)) return 0;
  return make_layout(cfg).total;
}

int lss_create(const lss_config* cfg, const void* const* tensors, int32_t n_tensors, void* workspace,
               size_t workspace_bytes, void* hip_stream, lss_engine** out) {
  lss_engine* e = nullptr;
  std::string why;
  if (!out) return create_fail(LSS_EINVAL, "create: null out");
  *out = nullptr;
  if (!cfg_valid(cfg, &why)) return create_fail(LSS_EINVAL, "create: " + why);
  if (!tensors || n_tensors != 3 + 9 * cfg->n_layers)
    return create_fail(LSS_EINVAL, "create: expected 3 + 9 * n_layers tensors");
  if (!workspace) return create_fail(LSS_EINVAL, "create: null workspace");
  for (int i = 0; i < n_tensors; ++i)
    if (!tensors[i] || ((uintptr_t)tensors[i] & 15))
      return create_fail(LSS_EINVAL, "create: tensor " + std::to_string(i) + " is null or not 16-byte aligned");
  if (((uintptr_t)workspace & 255)) return create_fail(LSS_EINVAL, "create: workspace not 256-byte aligned");
  const Layout lay = make_layout(cfg);
  if (workspace_bytes < lay.total) return create_fail(LSS_ECAPACITY, "create: workspace smaller than lss_workspace_bytes");

  e = new lss_engine();
  e->cfg = *cfg;
  e->lay = lay;
  e->stream = (hipStream_t)hip_stream;
  e->bf16 = cfg->dtype == LSS_BF16;
  e->kv16 = cfg->kv_dtype == LSS_BF16;
  {  // decode-GEMV grid: the compute units of the current device
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      e->gvl.ncu = ncu;
    e->gvl.gmax_cu = LSS_GEMV_WGS_PER_CU;
  }
  e->embed = tensors[0];
  e->final_norm = (const float*)tensors[1];
  e->lm_head = tensors[2];
  e->layers.resize(cfg->n_layers);
  for (int l = 0; l < cfg->n_layers; ++l) {
    const void* const* t = tensors + 3 + 9 * l;
    e->layers[l] = LayerW{(const float*)t[0], t[1], t[2], t[3], t[4], (const float*)t[5], t[6], t[7], t[8]};
  }
  char* ws = (char*)workspace;
  e->ws = ws;
  e->kc_all = ws + lay.kc; e->vc_all = ws + lay.vc;
  e->kc = e->kc_all; e->vc = e->vc_all;
  e->hs = (float*)(ws + lay.hs); e->hmid = (float*)(ws + lay.hmid);
  e->xa = ws + lay.xa; e->xb = ws + lay.xb; e->xc = ws + lay.xc;
  e->pa = (float*)(ws + lay.pa); e->pc = (float*)(ws + lay.pc);
  e->xs = (float*)(ws + lay.xs); e->qkv = (float*)(ws + lay.qkv);
  e->pgpart = (float*)(ws + lay.pgpart); e->rstd = (float*)(ws + lay.rstd);
  e->apart = (float*)(ws + lay.apart); e->aout = (float*)(ws + lay.aout);
  e->act = (float*)(ws + lay.act); e->logits = (float*)(ws + lay.logits); e->hpart = (float*)(ws + lay.hpart);
  e->rope = (float2*)(ws + lay.rope); e->target_all = (float*)(ws + lay.target); e->target = e->target_all;
  e->dpg[0] = (float*)(ws + lay.dpg0); e->dpg[1] = (float*)(ws + lay.dpg1); e->dpx = (float*)(ws + lay.dpx);
  e->dpdec = (float*)(ws + lay.dpdec); e->tok_all = (int32_t*)(ws + lay.tok); e->tok = e->tok_all;
  e->seqtok = (int32_t*)(ws + lay.seqtok);
  e->res_all = (HeadRes*)(ws + lay.res); e->res = e->res_all;
  e->dlogits = (float*)(ws + lay.dlogits); e->srec = (float*)(ws + lay.srec);
  e->q8 = (int8_t*)(ws + lay.q8);
  e->valid.assign(cfg->n_layers, 0u);
  e->nseq = lay.nseq;
  e->seqs.resize(e->nseq);
  for (auto& q : e->seqs) q.valid.assign(cfg->n_layers, 0u);
  {  // every workspace pointer must be set (a null one would be written by a kernel)
    const void* ptrs[] = {e->kc, e->vc, e->hs, e->hmid, e->xa, e->xb, e->xc, e->pa, e->pc, e->xs, e->qkv,
                          e->pgpart, e->rstd, e->apart, e->aout, e->act, e->logits, e->hpart, e->rope,
                          e->target, e->dpg[0], e->dpg[1], e->dpx, e->dpdec, e->tok, e->seqtok, e->res,
                          e->dlogits, e->srec, e->q8};
    for (const void* q : ptrs)
      if (!q) {
        lss_destroy(e);
        return create_fail(LSS_EINVAL, "create: workspace layout has a null buffer");
      }
  }

  hipError_t s = hipHostMalloc((void**)&e->hres_all, sizeof(HeadRes) * (e->nseq + 1), hipHostMallocDefault);
  e->hres = e->hres_all;
  if (s == hipSuccess)
    s = hipHostMalloc((void**)&e->hstage, ((size_t)cfg->max_seq + 64) * sizeof(int32_t), hipHostMallocDefault);
  if (s != hipSuccess) {
    lss_destroy(e);
    return create_fail(LSS_EHIP, std::string("create: hipHostMalloc: ") + hipGetErrorString(s));
  }
  // zero the workspace (stale KV rows past the committed length must be finite)
  fill_u32(e, ws, lay.total / 4, 0u);
  // rotary table: angle t * theta^(-2i/hd) in double, cos/sin rounded to float
  {
    const int half = cfg->head_dim / 2;
    std::vector<float2> tab((size_t)cfg->max_seq * half);
    for (int t = 0; t < cfg->max_seq; ++t)
      for (int i = 0; i < half; ++i) {
        const double ang = (double)t * std::pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim);
        tab[(size_t)t * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
      }
    s = hipMemcpyAsync(e->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice, e->stream);
    if (s == hipSuccess) s = hipStreamSynchronize(e->stream);
    if (s == hipSuccess) s = hipGetLastError();
    if (s != hipSuccess) {
      lss_destroy(e);
      return create_fail(LSS_EHIP, std::string("create: workspace setup: ") + hipGetErrorString(s));
    }
  }
  *out = e;
  return LSS_OK;
}

int lss_load_weights(const lss_config* cfg, const lss_tensor* tensors, int32_t n_tensors, void* workspace,
                     size_t workspace_bytes, void* hip_stream, lss_engine** out) {
  std::string why;
  if (!out) return create_fail(LSS_EINVAL, "load_weights: null out");
  *out = nullptr;
  if (!cfg_valid(cfg, &why)) return create_fail(LSS_EINVAL, "load_weights: " + why);
  if (!tensors || n_tensors != 3 + 9 * cfg->n_layers)
    return create_fail(LSS_EINVAL, "load_weights: expected 3 + 9 * n_layers tensors");
  const int64_t d = cfg->d_model, F = cfg->ffn_dim, V = cfg->vocab;
  const int64_t qd = (int64_t)cfg->n_heads * cfg->head_dim, kvd = (int64_t)cfg->n_kv_heads * cfg->head_dim;
  static const char* const kLayer[9] = {"attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down"};
  const int64_t layer_numel[9] = {d, qd * d, kvd * d, kvd * d, d * qd, d, F * d, F * d, d * F};
  std::vector<const void*> ptrs(n_tensors);
  for (int i = 0; i < n_tensors; ++i) {
    std::string name;
    int64_t numel;
    if (i < 3) {
      static const char* const kGlobal[3] = {"embed", "final_norm", "lm_head"};
      name = kGlobal[i];
      numel = i == 1 ? d : V * d;
    } else {
      const int l = (i - 3) / 9, j = (i - 3) % 9;
      name = "layers." + std::to_string(l) + "." + kLayer[j];
      numel = layer_numel[j];
    }
    const lss_tensor& t = tensors[i];
    if (!t.name || name != t.name)
      return create_fail(LSS_EINVAL, "load_weights: tensor " + std::to_string(i) + " must be '" + name + "', got '" +
                                         (t.name ? t.name : "(null)") + "'");
    if (t.numel != numel)
      return create_fail(LSS_EINVAL, "load_weights: '" + name + "' has " + std::to_string(t.numel) +
                                         " elements, the config implies " + std::to_string(numel));
    ptrs[i] = t.dev_ptr;
  }
  return lss_create(cfg, ptrs.data(), n_tensors, workspace, workspace_bytes, hip_stream, out);
}

void lss_destroy(lss_engine* e) {
  if (!e) return;
  (void)hipStreamSynchronize(e->stream);
  for (auto ev : e->ev_start) (void)hipEventDestroy(ev);
  for (auto ev : e->ev_stop) (void)hipEventDestroy(ev);
  if (e->hres_all) (void)hipHostFree(e->hres_all);
  if (e->hstage) (void)hipHostFree(e->hstage);
  delete e;
}

const char* lss_last_error(const lss_engine* e) { return e ? e->err.c_str() : g_create_err.c_str(); }

int32_t lss_seq_len(const lss_engine* e) { return e ? e->p : -1; }

size_t lss_w8_bytes(const lss_config* cfg) {
  if (!cfg_valid(cfg, nullptr)) return 0;
  return w8_layout(cfg, nullptr);
}

int lss_attach_w8(lss_engine* e, void* buf, size_t bytes) {
  if (!e) return LSS_EINVAL;
  const lss_config* c = &e->cfg;
  std::vector<std::array<size_t, 14>> offs;
  const size_t need = w8_layout(c, &offs);
  if (!buf || ((uintptr_t)buf & 255)) return fail(e, LSS_EINVAL, "attach_w8: null or unaligned buffer");
  if (bytes < need) return fail(e, LSS_ECAPACITY, "attach_w8: buffer smaller than lss_w8_bytes");
  int n[7], k[7];
  w8_shapes(c, n, k);
  std::vector<LayerW8> w8(c->n_layers);
  char* b = (char*)buf;
  for (int l = 0; l < c->n_layers; ++l) {
    const LayerW& w = e->layers[l];
    const void* src[7] = {w.wq, w.wk, w.wv, w.wo, w.wg, w.wu, w.wd};
    for (int i = 0; i < 7; ++i) {
      int8_t* q = (int8_t*)(b + offs[l][i]);
      float* sc = (float*)(b + offs[l][7 + i]);
      if (e->bf16)
        hipLaunchKernelGGL(k_quant_w8<uint16_t>, dim3(n[i]), dim3(256), 0, e->stream, (const uint16_t*)src[i], k[i], q, sc);
      else
        hipLaunchKernelGGL(k_quant_w8<float>, dim3(n[i]), dim3(256), 0, e->stream, (const float*)src[i], k[i], q, sc);
      w8[l].q[i] = q;
      w8[l].s[i] = sc;
    }
  }
  int rc = check_launch(e, "attach_w8");
  if (rc) return rc;
  HIPCHK(hipStreamSynchronize(e->stream));
  e->w8 = std::move(w8);
  return LSS_OK;
}

int lss_op_w8_quantize(const void* w, int32_t dtype, int32_t rows, int32_t k, int8_t* q, float* scale, void* stream) {
  if (!w || !q || !scale || rows < 0 || k < 0 || (dtype != LSS_F32 && dtype != LSS_BF16)) return LSS_EINVAL;
  if (rows == 0) return LSS_OK;
  if (dtype == LSS_BF16)
    hipLaunchKernelGGL(k_quant_w8<uint16_t>, dim3(rows), dim3(256), 0, (hipStream_t)stream, (const uint16_t*)w, k, q, scale);
  else
    hipLaunchKernelGGL(k_quant_w8<float>, dim3(rows), dim3(256), 0, (hipStream_t)stream, (const float*)w, k, q, scale);
  return hipGetLastError() == hipSuccess ? LSS_OK : LSS_EHIP;
}

int lss_op_w8a8_gemv(const int8_t* wq, const float* wscale, int32_t n, int32_t k, const int8_t* xq,
                     const float* xscale, float* y, void* stream) {
  if (!wq || !wscale || !xq || !xscale || !y || n < 1 || k < 16 || n % 16 || k % 16 || k > G8_KMAX)
    return LSS_EINVAL;
  if (((uintptr_t)wq & 15) || ((uintptr_t)xq & 15)) return LSS_EINVAL;
  GemmArgs ga{};
  ga.w[0] = ga.w[1] = ga.w[2] = wq;
  ga.nseg[0] = n;
  ga.wsc[0] = ga.wsc[1] = ga.wsc[2] = wscale;
  ga.N = n; ga.K = k; ga.M = 1; ga.xq = xq; ga.xs = xscale; ga.Y = y; ga.ldy = n;
  hipLaunchKernelGGL((k_gemv8<float, EPI_STORE, 8>), dim3(n / G8_TR), dim3(G8_THREADS), 0, (hipStream_t)stream, ga);
  return hipGetLastError() == hipSuccess ? LSS_OK : LSS_EHIP;
}

int lss_op_w8a8_gemv_f32(const int8_t* wq, const float* wscale, int32_t n, int32_t k, const float* x, float* y,
                         void* stream) {
  if (!wq || !wscale || !x || !y || n < 1 || k < 16 || n % 16 || k % 16 || k > G8_KMAX) return LSS_EINVAL;
  if ((uintptr_t)wq & 15) return LSS_EINVAL;
  GemmArgs ga{};
  ga.w[0] = ga.w[1] = ga.w[2] = wq;
  ga.nseg[0] = n;
  ga.wsc[0] = ga.wsc[1] = ga.wsc[2] = wscale;
  ga.N = n; ga.K = k; ga.M = 1; ga.A = x; ga.lda = k; ga.scale = SCALE_NONE; ga.Y = y; ga.ldy = n;
  const dim3 grid(n / G8_TR), block(G8_THREADS);
  const hipStream_t s = (hipStream_t)stream;
  const int per = (k + G8_THREADS - 1) / G8_THREADS;
  if (per <= 8) hipLaunchKernelGGL((k_gemv8<float, EPI_STORE, 8>), grid, block, 0, s, ga);
  else if (per <= 16) hipLaunchKernelGGL((k_gemv8<float, EPI_STORE, 16>), grid, block, 0, s, ga);
  else if (per <= 32) hipLaunchKernelGGL((k_gemv8<float, EPI_STORE, 32>), grid, block, 0, s, ga);
  else hipLaunchKernelGGL((k_gemv8<float, EPI_STORE, 64>), grid, block, 0, s, ga);
  return hipGetLastError() == hipSuccess ? LSS_OK : LSS_EHIP;
}

int lss_set_sampling(lss_engine* e, float temperature, uint64_t seed) {
  if (!e) return LSS_EINVAL;
  if (!(temperature >= 0.f) || !std::isfinite(temperature))
    return fail(e, LSS_EINVAL, "set_sampling: temperature must be finite and >= 0");
  seq_save(e);
  for (const SeqState& q : e->seqs)
    if (q.win > 0 || q.pending_accept)
      return fail(e, LSS_ESTATE, "set_sampling: a draft window or verify is pending (on some sequence)");
  const float inv = temperature > 0.f ? 1.0f / temperature : 0.f;
  if (temperature > 0.f && !std::isfinite(inv)) return fail(e, LSS_EINVAL, "set_sampling: temperature too small");
  e->inv_t = inv;
  e->seed = seed;
  return LSS_OK;
}

int lss_set_gemv_grid(lss_engine* e, int32_t wgs_per_cu) {
  if (!e) return LSS_EINVAL;
  if (wgs_per_cu < 0 || wgs_per_cu > 8) return fail(e, LSS_EINVAL, "set_gemv_grid: wgs_per_cu must be in [0, 8]");
  e->gvl.gmax_cu = wgs_per_cu;
  return LSS_OK;
}

int lss_set_decode_kernel(lss_engine* e, int32_t kind) {
  if (!e) return LSS_EINVAL;
  if (kind < 0 || kind > 2) return fail(e, LSS_EINVAL, "set_decode_kernel: kind must be 0, 1 or 2");
  if (e->win > 0 || e->pending_accept)
    return fail(e, LSS_ESTATE, "set_decode_kernel: a draft window or verify is pending");
  e->decode_mfma = kind >= 1;
  e->draft_mfma = kind == 1;
  return LSS_OK;
}

int lss_prefill(lss_engine* e, const int32_t* tokens, int32_t n, int32_t* t0_out) {
  if (!e) return LSS_EINVAL;
  const auto& c = e->cfg;
  if (!tokens || n < 1) return fail(e, LSS_EINVAL, "prefill: empty prompt");
  if (n + 1 > c.max_seq) return fail(e, LSS_ECAPACITY, "prefill: prompt exceeds max_seq - 1");
  for (int i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= c.vocab) return fail(e, LSS_EINVAL, "prefill: token id out of range");
  std::memcpy(e->hstage, tokens, sizeof(int32_t) * n);
  HIPCHK(hipMemcpyAsync(e->seqtok, e->hstage, sizeof(int32_t) * n, hipMemcpyHostToDevice, e->stream));
  const int R = c.max_rows;
  int last_m = 0;
  for (int c0 = 0; c0 < n; c0 += R) {
    const int M = std::min(R, n - c0);
    forward_rows(e, e->seqtok + c0, M, c0);
    last_m = M - 1;
  }
  head(e, last_m, 1, 0, n - 1, false);
  hipLaunchKernelGGL(k_accept, dim3(1), dim3(1), 0, e->stream, e->res, 0, e->tok,
                     e->inv_t > 0.f ? 1 : 0);  // tok[0] = argmax, or the draw
  hipLaunchKernelGGL(k_gather_target, dim3(c.n_layers + 1), dim3(256), 0, e->stream, e->hs, R, c.d_model,
                     (const HeadRes*)nullptr, last_m, e->target);
  int rc = check_launch(e, "prefill");
  if (rc) return rc;
  rc = sync_res(e);
  if (rc) return rc;
  e->p = n;
  e->win = 0;
  std::fill(e->valid.begin(), e->valid.end(), 0u);
  e->have_seq = true;
  e->pending_accept = false;
  e->have_target = true;
  e->target_pos = n - 1;
  if (t0_out) *t0_out = e->hres->bonus;
  return LSS_OK;
}

int lss_draft(lss_engine* e, const uint8_t* mask, int32_t quant, int32_t k, float exit_tau, int32_t* tokens_out,
              int32_t* k_done) {
  if (!e) return LSS_EINVAL;
  const GemvScope gv(e, true);
  const auto& c = e->cfg;
  if (!e->have_seq || e->pending_accept) return fail(e, LSS_ESTATE, "draft: needs a prefilled sequence and no pending accept");
  if (!mask || k < 0 || quant < 0 || quant > 2) return fail(e, LSS_EINVAL, "draft: bad arguments");
  if (quant == 2 && e->w8.empty()) return fail(e, LSS_ESTATE, "draft: int8 weights not attached (lss_attach_w8)");
  if (e->tree > 0) return fail(e, LSS_ESTATE, "draft: a tree window is pending");
  if (k > 0 && !tokens_out) return fail(e, LSS_EINVAL, "draft: null tokens_out");
  const int win_cap = std::min(kWinMax, c.max_rows - 1);
  if (e->win + k > win_cap) return fail(e, LSS_ECAPACITY, "draft: window would exceed its capacity");
  if (e->p + e->win + k + 1 > c.max_seq) return fail(e, LSS_ECAPACITY, "draft: KV capacity exceeded");
  const int start = e->win;
  int done = 0;
  for (int s = 0; s < k; ++s) {
    const int slot = e->win;
    const int pos = e->p + slot;
    embed(e, e->tok + slot, 1, hs_row(e, 0, 0), next_gain(e, mask, -1));
    const float* h = hs_row(e, 0, 0);
    for (int l = 0; l < c.n_layers; ++l) {
      if (mask[l]) continue;
      e->valid[l] |= 1u << slot;
      layer_forward(e, l, 1, h, e->xa, e->pa, hs_row(e, l + 1, 0), next_gain(e, mask, l), MODE_DRAFT, pos, quant);
      h = hs_row(e, l + 1, 0);
    }
    head(e, 0, 1, slot, pos, true);
    hipLaunchKernelGGL(k_draft_commit, dim3(1), dim3(1), 0, e->stream, e->res, slot, e->tok, e->inv_t > 0.f ? 1 : 0);
    e->win++;
    done++;
    if (exit_tau > 0.f) {
      int rc = check_launch(e, "draft");
      if (rc) return rc;
      rc = sync_res(e);
      if (rc) return rc;
      if (e->hres->pmax[slot] < exit_tau) break;
    }
  }
  int rc = check_launch(e, "draft");
  if (rc) return rc;
  if (done > 0) {
    rc = sync_res(e);
    if (rc) return rc;
    const int32_t* drawn = e->inv_t > 0.f ? e->hres->sample : e->hres->argmax;
    for (int i = 0; i < done; ++i) tokens_out[i] = drawn[start + i];
  }
  if (k_done) *k_done = done;
  return LSS_OK;
}

int lss_draft_tree_levels(lss_engine* e, const uint8_t* masks, const int32_t* quants, int32_t B, int32_t D,
                          int32_t* tokens_out) {
  if (!e) return LSS_EINVAL;
  const GemvScope gv(e, true);
  const auto& c = e->cfg;
  const int L = c.n_layers;
  if (!e->have_seq || e->pending_accept || e->win != 0)
    return fail(e, LSS_ESTATE, "draft_tree: needs a prefilled sequence, no pending accept and an empty window");
  if (!masks || !quants || !tokens_out || B < 1 || B > TOPB_MAX || B > c.vocab || D < 1)
    return fail(e, LSS_EINVAL, "draft_tree: bad arguments (1 <= B <= 8, D >= 1)");
  if (e->inv_t > 0.f) return fail(e, LSS_EINVAL, "draft_tree: tree acceptance is greedy; sampling is on");
  const long nodes = (long)B * D;
  if (nodes > LSS_TREE_NODES_MAX || nodes + 1 > c.max_rows || nodes > kWinMax)
    return fail(e, LSS_ECAPACITY, "draft_tree: B * D above LSS_TREE_NODES_MAX or max_rows - 1");
  for (int j = 0; j < D; ++j) {
    if (quants[j] < 0 || quants[j] > 2) return fail(e, LSS_EINVAL, "draft_tree: quant must be 0, 1 or 2");
    if (quants[j] == 2 && e->w8.empty()) return fail(e, LSS_ESTATE, "draft_tree: int8 weights not attached");
  }
  if (e->p + nodes + 1 > c.max_seq) return fail(e, LSS_ECAPACITY, "draft_tree: KV capacity exceeded");
  static_assert(LSS_TREE_NODES_MAX < ATT_TREE_NODES, "tree nodes must fit the attention kernel's node arrays");
  static_assert(LSS_TREE_NODES_MAX < 32, "tree depths must fit the per-layer valid bits");
  // the draft row of the pending token (slot 0, position p) with the first
  // depth's level, then its top B as the branches' first nodes (window
  // slots 1 + b D)
  const uint8_t* m0 = masks;
  embed(e, e->tok, 1, hs_row(e, 0, 0), next_gain(e, m0, -1));
  const float* h = hs_row(e, 0, 0);
  for (int l = 0; l < L; ++l) {
    if (m0[l]) continue;
    e->valid[l] |= 1u;
    layer_forward(e, l, 1, h, e->xa, e->pa, hs_row(e, l + 1, 0), next_gain(e, m0, l), MODE_DRAFT, e->p, quants[0]);
    h = hs_row(e, l + 1, 0);
  }
  head(e, 0, 1, 0, e->p, true);
  hipLaunchKernelGGL(k_topb, dim3(1), dim3(TOPB_THREADS), 0, e->stream, (const float*)e->logits, c.vocab, B, D, e->tok);
  // depth j = 1 .. D - 1: node j of branches b0 .. b0 + M - 1 (window slots
  // 1 + b D + j - 1) through the level of depth j + 1, their argmax nodes
  // j + 1.  A layer sees position p + i (the pending token, or node i of the
  // row's branch) only where the pass over depth i ran it: valid bit i of
  // the layer, set here for depth j.  Int8 weights draft one row at a time,
  // so one branch per pass there.
  e->tree_D = D;
  auto step = [&](int j, int b0, int M) {
    const uint8_t* mk = masks + (size_t)j * L;
    e->tree_step = j;
    e->tree_b0 = b0;
    embed(e, e->tok + 1 + b0 * D + j - 1, M, hs_row(e, 0, 0), next_gain(e, mk, -1), D);
    const float* hh = hs_row(e, 0, 0);
    for (int l = 0; l < L; ++l) {
      if (mk[l]) continue;
      e->valid[l] |= 1u << j;
      layer_forward(e, l, M, hh, e->xa, e->pa, hs_row(e, l + 1, 0), next_gain(e, mk, l), MODE_TREE_DRAFT, e->p,
                    quants[j]);
      hh = hs_row(e, l + 1, 0);
    }
    head(e, 0, M, b0, e->p + j, true);
  };
  for (int j = 1; j < D; ++j) {
    if (quants[j] == 2)
      for (int b = 0; b < B; ++b) step(j, b, 1);
    else
      step(j, 0, B);
    hipLaunchKernelGGL(k_tree_draft_commit, dim3(1), dim3(64), 0, e->stream, (const HeadRes*)e->res, B, D, j, e->tok);
  }
  e->tree_step = 0;
  e->tree_b0 = 0;
  int rc = check_launch(e, "draft_tree");
  if (rc) return rc;
  HIPCHK(hipMemcpyAsync(e->hstage, e->tok + 1, sizeof(int32_t) * nodes, hipMemcpyDeviceToHost, e->stream));
  HIPCHK(hipStreamSynchronize(e->stream));
  std::memcpy(tokens_out, e->hstage, sizeof(int32_t) * nodes);
  e->win = (int)nodes;
  e->tree = B;
  return LSS_OK;
}

int lss_draft_tree(lss_engine* e, const uint8_t* mask, int32_t quant, int32_t B, int32_t D, int32_t* tokens_out) {
  if (!e) return LSS_EINVAL;
  const int L = e->cfg.n_layers;
  const bool ok = mask && D >= 1 && D <= kWinMax;
  std::vector<uint8_t> masks(ok ? (size_t)D * L : 0);
  std::vector<int32_t> quants(ok ? D : 0, quant);
  for (int j = 0; ok && j < D; ++j) std::copy(mask, mask + L, masks.begin() + (size_t)j * L);
  return lss_draft_tree_levels(e, ok ? masks.data() : nullptr, ok ? quants.data() : nullptr, B, D, tokens_out);
}

int lss_verify(lss_engine* e, const int32_t* drafts, int32_t k) {
  if (!e) return LSS_EINVAL;
  const GemvScope gv(e);
  const auto& c = e->cfg;
  if (!e->have_seq || e->pending_accept) return fail(e, LSS_ESTATE, "verify: needs a prefilled sequence and no pending accept");
  const bool samp = e->inv_t > 0.f;
  if (drafts) {
    if (samp && k > 0) return fail(e, LSS_EINVAL, "verify: host-forced drafts need greedy mode (no draft distribution)");
    if (k < 0 || k > std::min(kWinMax, c.max_rows - 1)) return fail(e, LSS_ECAPACITY, "verify: k exceeds the window capacity");
    for (int i = 0; i < k; ++i)
      if (drafts[i] < 0 || drafts[i] >= c.vocab) return fail(e, LSS_EINVAL, "verify: token id out of range");
  } else {
    if (k != e->win) return fail(e, LSS_EINVAL, "verify: k must equal the pending window length");
  }
  if (e->p + k + 1 > c.max_seq) return fail(e, LSS_ECAPACITY, "verify: KV capacity exceeded");
  if (e->tree > 0 && drafts)
    return fail(e, LSS_EINVAL, "verify: a tree window is pending; verify it with drafts == NULL");
  // every check is done: only now may host-forced drafts replace the window
  if (drafts && k > 0) {
    std::memcpy(e->hstage, drafts, sizeof(int32_t) * k);
    HIPCHK(hipMemcpyAsync(e->tok + 1, e->hstage, sizeof(int32_t) * k, hipMemcpyHostToDevice, e->stream));
  }
  const int M = k + 1;
  if (e->tree > 0) {                                   // width-B tree: one pass, tree mask
    forward_rows(e, e->tok, M, e->p, MODE_TREE);
    head(e, 0, M, 0, e->p, false);
    hipLaunchKernelGGL(k_accept_tree, dim3(1), dim3(1), 0, e->stream, e->res, e->tree, e->tree_D, e->tok);
    const dim3 fg(c.n_layers, c.n_kv_heads);
    if (e->kv16)
      hipLaunchKernelGGL(k_tree_kv_fix<uint16_t>, fg, dim3(256), 0, e->stream, (const HeadRes*)e->res, e->tree_D,
                         (uint16_t*)e->kc, (uint16_t*)e->vc, c.n_kv_heads, c.max_seq, c.head_dim, e->p);
    else
      hipLaunchKernelGGL(k_tree_kv_fix<float>, fg, dim3(256), 0, e->stream, (const HeadRes*)e->res, e->tree_D,
                         (float*)e->kc, (float*)e->vc, c.n_kv_heads, c.max_seq, c.head_dim, e->p);
    hipLaunchKernelGGL(k_gather_target, dim3(c.n_layers + 1), dim3(256), 0, e->stream, e->hs, c.max_rows,
                       c.d_model, (const HeadRes*)e->res, 0, e->target);
    const int rc = check_launch(e, "verify");
    if (rc) return rc;
    e->win = k;
    e->verify_rows = M;
    e->pending_accept = true;
    return LSS_OK;
  }
  forward_rows(e, e->tok, M, e->p);
  head(e, 0, M, 0, e->p, false);
  if (samp && k > 0) {
    const int nrec = (c.vocab + SPEC_RES_PER_WG - 1) / SPEC_RES_PER_WG;
    hipLaunchKernelGGL(k_spec_residual, dim3(nrec), dim3(SPEC_RES_THREADS), 0, e->stream, (const float*)e->logits,
                       (const float*)e->dlogits, c.vocab, (const HeadRes*)e->res, (const int32_t*)e->tok, k, e->inv_t,
                       e->seed, e->p, e->srec);
    hipLaunchKernelGGL(k_spec_final, dim3(1), dim3(SPEC_FIN_THREADS), 0, e->stream, (const float*)e->logits,
                       (const float*)e->dlogits, c.vocab, e->res, e->tok, k, e->inv_t, e->seed, e->p,
                       (const float*)e->srec, nrec);
  } else {
    hipLaunchKernelGGL(k_accept, dim3(1), dim3(1), 0, e->stream, e->res, k, e->tok, samp ? 1 : 0);
  }
  hipLaunchKernelGGL(k_gather_target, dim3(c.n_layers + 1), dim3(256), 0, e->stream, e->hs, c.max_rows,
                     c.d_model, (const HeadRes*)e->res, 0, e->target);
  const int rc = check_launch(e, "verify");
  if (rc) return rc;
  e->win = k;
  e->verify_rows = M;
  e->pending_accept = true;
  return LSS_OK;
}

int lss_accept_and_rollback(lss_engine* e, int32_t* n_accepted, int32_t* bonus, int32_t* accepted_out) {
  if (!e) return LSS_EINVAL;
  if (!e->pending_accept) return fail(e, LSS_ESTATE, "accept: no verify pending");
  const int rc = sync_res(e);
  if (rc) return rc;
  const int n = e->hres->n;
  if (n_accepted) *n_accepted = n;
  if (bonus) *bonus = e->hres->bonus;
  if (accepted_out)
    for (int i = 0; i <= n; ++i) accepted_out[i] = e->hres->emit[i];
  e->target_pos = e->p + n;
  e->have_target = true;
  e->p += n + 1;
  e->win = 0;
  e->tree = 0;
  e->tree_D = 1;
  std::fill(e->valid.begin(), e->valid.end(), 0u);
  e->pending_accept = false;
  return LSS_OK;
}

int lss_select_layers_dp(lss_engine* e, int32_t S, uint8_t* mask_out, float* score_out) {
  if (!e) return LSS_EINVAL;
  return lss_select_layers_dp_exit(e, S, e->cfg.n_layers, mask_out, score_out);
}

int lss_select_layers_dp_exit(lss_engine* e, int32_t S, int32_t Le, uint8_t* mask_out, float* score_out) {
  if (!e) return LSS_EINVAL;
  const auto& c = e->cfg;
  const int L = c.n_layers, d = c.d_model;
  if (!mask_out || Le < 0 || Le > L || S < 0 || S > Le) return fail(e, LSS_EINVAL, "select_layers_dp: bad n_skip / n_layers_eff");
  if (!e->have_target || e->pending_accept) return fail(e, LSS_ESTATE, "select_layers_dp: no target state");
  if (std::min(S, Le - S) + 1 > c.max_rows) return fail(e, LSS_ECAPACITY, "select_layers_dp: more DP rows than max_rows");
  auto lo = [&](int i) { return std::max(0, S - (Le - i)); };
  auto hi = [&](int i) { return std::min(i, S); };
  const int tstar = e->target_pos;
  fill_u32(e, e->dpdec, (size_t)(L + 1) * (L + 1) * 3, 0x7fc00000u);
  HIPCHK(hipMemcpyAsync(e->dpg[0], e->target, sizeof(float) * d, hipMemcpyDeviceToDevice, e->stream));
  if (Le > 0) prep_rows(e, e->dpg[0], 1, e->layers[0].attn_norm, e->xa, e->pa);
  const int T = d / 16;
  int cur = 0;
  for (int i = 1; i <= Le; ++i) {
    const int lo_p = lo(i - 1), hi_p = hi(i - 1), lo_i = lo(i), hi_i = hi(i);
    const int ex_lo = std::max(lo_i, lo_p), ex_hi = std::min(hi_i, hi_p);
    const int ne = ex_hi - ex_lo + 1;
    const int off = ex_lo - lo_p;     // first executed row among the stage's input rows
    if (ne > 0)
      layer_forward(e, i - 1, ne, e->dpg[cur] + (size_t)off * d, xrow(e->xa, d, off), e->pa + (size_t)off * T,
                    e->dpx, nullptr, MODE_DP, tstar, 0);
    const float* g = i < Le ? e->layers[i].attn_norm : nullptr;
    void* xo = i < Le ? e->xa : nullptr;
    if (e->bf16)
      hipLaunchKernelGGL(k_dp_select<uint16_t>, dim3(hi_i - lo_i + 1), dim3(PREP_THREADS), 0, e->stream, e->dpx, ex_lo, ex_hi,
                         e->dpg[cur], lo_p, hi_p, e->target + (size_t)i * d, d, lo_i, e->dpg[cur ^ 1],
                         e->dpdec + (size_t)i * (L + 1) * 3, g, xo, e->pa);
    else
      hipLaunchKernelGGL(k_dp_select<float>, dim3(hi_i - lo_i + 1), dim3(PREP_THREADS), 0, e->stream, e->dpx, ex_lo, ex_hi,
                         e->dpg[cur], lo_p, hi_p, e->target + (size_t)i * d, d, lo_i, e->dpg[cur ^ 1],
                         e->dpdec + (size_t)i * (L + 1) * 3, g, xo, e->pa);
    cur ^= 1;
  }
  int rc = check_launch(e, "select_layers_dp");
  if (rc) return rc;
  std::vector<float> dec((size_t)(L + 1) * (L + 1) * 3);
  HIPCHK(hipMemcpyAsync(dec.data(), e->dpdec, dec.size() * sizeof(float), hipMemcpyDeviceToHost, e->stream));
  HIPCHK(hipStreamSynchronize(e->stream));
  for (int l = 0; l < L; ++l) mask_out[l] = l >= Le ? 1 : 0;
  int j = S;
  float score = 1.f;
  if (Le > 0) {
    const float* f = &dec[((size_t)Le * (L + 1) + S) * 3];
    score = f[0] != 0.f ? f[1] : f[2];
  }
  for (int i = Le; i >= 1; --i) {
    const float take = dec[((size_t)i * (L + 1) + j) * 3];
    if (take != 0.f) { mask_out[i - 1] = 1; --j; }
  }
  if (j != 0) return fail(e, LSS_EHIP, "select_layers_dp: inconsistent back-pointers");
  if (score_out) *score_out = score;
  return LSS_OK;
}

int lss_read_logits(lss_engine* e, int32_t rows, float* host_out) {
  if (!e || !host_out || rows < 1 || rows > e->logits_rows) return fail(e, LSS_EINVAL, "read_logits: bad rows");
  HIPCHK(hipMemcpyAsync(host_out, e->logits, sizeof(float) * rows * (size_t)e->cfg.vocab, hipMemcpyDeviceToHost,
                        e->stream));
  HIPCHK(hipStreamSynchronize(e->stream));
  return LSS_OK;
}

int lss_read_states(lss_engine* e, int32_t row, float* host_out) {
  if (!e || !host_out || row < 0 || row >= e->cfg.max_rows) return fail(e, LSS_EINVAL, "read_states: bad row");
  const auto& c = e->cfg;
  for (int l = 0; l <= c.n_layers; ++l)
    HIPCHK(hipMemcpyAsync(host_out + (size_t)l * c.d_model, hs_row(e, l, row), sizeof(float) * c.d_model,
                          hipMemcpyDeviceToHost, e->stream));
  HIPCHK(hipStreamSynchronize(e->stream));
  return LSS_OK;
}

int lss_read_dp_decisions(lss_engine* e, float* host_out) {
  if (!e || !host_out) return LSS_EINVAL;
  const size_t n = (size_t)(e->cfg.n_layers + 1) * (e->cfg.n_layers + 1) * 3;
  HIPCHK(hipMemcpyAsync(host_out, e->dpdec, n * sizeof(float), hipMemcpyDeviceToHost, e->stream));
  HIPCHK(hipStreamSynchronize(e->stream));
  return LSS_OK;
}

int lss_op_quantize_rows(const float* x, int32_t rows, int32_t n, int8_t* q, float* scale, void* stream) {
  if (!x || !q || !scale || rows < 0 || n < 0) return LSS_EINVAL;
  if (rows == 0 || n == 0) {
    if (rows > 0 && n == 0)
      hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(64), 0, (hipStream_t)stream, (uint32_t*)scale, (size_t)rows, 0u);
    return hipGetLastError() == hipSuccess ? LSS_OK : LSS_EHIP;
  }
  hipLaunchKernelGGL(k_quant_rows<float>, dim3(rows), dim3(256), 0, (hipStream_t)stream, x, n, n, (void*)nullptr,
                     scale, q);
  return hipGetLastError() == hipSuccess ? LSS_OK : LSS_EHIP;
}

// ---------------------------------------------------------------- stand-alone greedy acceptance
// Scratch of the allocation-free form: per-chunk records of up to
// LSS_ACCEPT_ROWS_MAX rows of LSS_ACCEPT_VOCAB_MAX logits (32 KB).  Every
// GPU the library runs on holds its own copy until the process ends; host
// code must use the address hipGetSymbolAddress gives for the current
// device, never the array's name (a host-side stand-in).
static __device__ __align__(256) AccRec scratch[LSS_ACCEPT_ROWS_MAX * (LSS_ACCEPT_VOCAB_MAX / ACC_CH)];

}  // extern "C" (the helpers below have C++ linkage)
namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[LSS_MAX_DEVICES] = {};

// this device's address of `scratch`, looked up once per device
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= LSS_MAX_DEVICES)
    return create_fail(LSS_EHIP, "accept_greedy_noalloc: no current device (or device id >= 64)");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t s = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s != hipSuccess || !p)
      return create_fail(LSS_EHIP, std::string("accept_greedy_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(s));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LSS_OK;
}

size_t accept_records(int32_t rows, int32_t vocab) {
  return (size_t)rows * ((vocab + ACC_CH - 1) / ACC_CH) * sizeof(AccRec);
}

int accept_launch(const float* logits, int32_t rows, int32_t vocab, const int32_t* drafts, int32_t* result,
                  AccRec* rec, hipStream_t s) {
  const int nchunk = (vocab + ACC_CH - 1) / ACC_CH;
  hipLaunchKernelGGL(k_argmax_chunks, dim3(nchunk, rows), dim3(ACC_THREADS), 0, s, logits, vocab, rec, nchunk);
  hipLaunchKernelGGL(k_accept_records, dim3(1), dim3(ACC_THREADS), 0, s, (const AccRec*)rec, nchunk, rows, vocab,
                     drafts, result);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return create_fail(LSS_EHIP, std::string("accept_greedy: launch: ") + hipGetErrorString(e));
  return LSS_OK;
}

int accept_args(const float* logits, int32_t rows, int32_t vocab, const int32_t* drafts, int32_t* result) {
  if (!logits || !result || (rows > 1 && !drafts)) return create_fail(LSS_EINVAL, "accept_greedy: null pointer");
  if (rows < 1 || rows > LSS_ACCEPT_ROWS_MAX || vocab < 1)
    return create_fail(LSS_EINVAL, "accept_greedy: rows must be in [1, 64], vocab >= 1");
  return LSS_OK;
}

}  // namespace
extern "C" {

size_t lss_op_accept_greedy_workspace_bytes(int32_t rows, int32_t vocab) {
  if (rows < 1 || rows > LSS_ACCEPT_ROWS_MAX || vocab < 1) return 0;
  return accept_records(rows, vocab);
}

int lss_op_accept_greedy(const float* logits, int32_t rows, int32_t vocab, const int32_t* drafts, int32_t* result,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int rc = accept_args(logits, rows, vocab, drafts, result);
  if (rc) return rc;
  if (!workspace) return create_fail(LSS_EINVAL, "accept_greedy: null workspace");
  if (workspace_bytes < accept_records(rows, vocab))
    return create_fail(LSS_ECAPACITY, "accept_greedy: workspace smaller than lss_op_accept_greedy_workspace_bytes");
  return accept_launch(logits, rows, vocab, drafts, result, (AccRec*)workspace, (hipStream_t)stream);
}

int lss_op_accept_greedy_noalloc(const float* logits, int32_t rows, int32_t vocab, const int32_t* drafts,
                                 int32_t* result, void* stream) {
  int rc = accept_args(logits, rows, vocab, drafts, result);
  if (rc) return rc;
  if (vocab > LSS_ACCEPT_VOCAB_MAX)
    return create_fail(LSS_ECAPACITY, "accept_greedy_noalloc: vocab above LSS_ACCEPT_VOCAB_MAX (262144); use "
                                      "lss_op_accept_greedy with a workspace");
  void* p = nullptr;
  rc = scratch_ptr(&p);
  if (rc) return rc;
  return accept_launch(logits, rows, vocab, drafts, result, (AccRec*)p, (hipStream_t)stream);
}

// ---------------------------------------------------------------- several sequences
int lss_seq_select(lss_engine* e, int32_t seq) {
  if (!e) return LSS_EINVAL;
  if (seq < 0 || seq >= e->nseq) return fail(e, LSS_EINVAL, "seq_select: index out of [0, max_seqs)");
  if (seq == e->cur) return LSS_OK;
  if (e->inv_t > 0.f && e->win > 0 && !e->pending_accept)
    return fail(e, LSS_ESTATE, "seq_select: sampling keeps one draft-distribution buffer; verify this window first");
  seq_save(e);
  seq_load(e, seq);
  return LSS_OK;
}

namespace {

// distinct sequence indices in range
bool seqs_valid(const lss_engine* e, int n, const int32_t* seqs) {
  if (n < 1 || n > e->nseq || !seqs) return false;
  std::vector<char> seen(e->nseq, 0);
  for (int i = 0; i < n; ++i) {
    if (seqs[i] < 0 || seqs[i] >= e->nseq || seen[seqs[i]]) return false;
    seen[seqs[i]] = 1;
  }
  return true;
}

// one batched draft step: one row per listed sequence (window slot win, at
// position p + win) through the layers mask keeps; the argmax becomes the
// slot's drafted token
void batch_draft_step(lss_engine* e, const std::vector<int>& sq, const uint8_t* mask, int quant) {
  const auto& c = e->cfg;
  const int M = (int)sq.size();
  RowTok rt{};
  BatchRows br{};
  br.n = M;
  e->pass.clear();
  for (int m = 0; m < M; ++m) {
    const SeqState& st = e->seqs[sq[m]];
    rt.off[m] = sq[m] * kTokSlots + st.win;
    br.seq[m] = sq[m];
    br.slot[m] = st.win;
    e->pass.push_back(PassSeq{sq[m], m, 1, st.p + st.win});
  }
  embed_rows(e, rt, M, hs_row(e, 0, 0), next_gain(e, mask, -1));
  const float* h = hs_row(e, 0, 0);
  for (int l = 0; l < c.n_layers; ++l) {
    if (mask[l]) continue;
    for (int m = 0; m < M; ++m) e->seqs[sq[m]].valid[l] |= 1u << e->seqs[sq[m]].win;
    layer_forward(e, l, M, h, e->xa, e->pa, hs_row(e, l + 1, 0), next_gain(e, mask, l), MODE_BATCH_DRAFT, 0, quant);
    h = hs_row(e, l + 1, 0);
  }
  HeadRes* bres = e->res_all + e->nseq;
  head(e, 0, M, 0, 0, true, bres);
  hipLaunchKernelGGL(k_draft_commit_b, dim3(1), dim3(BATCH_ROWS_MAX), 0, e->stream, (const HeadRes*)bres, br,
                     e->res_all, e->tok_all, kTokSlots);
  for (int m = 0; m < M; ++m) e->seqs[sq[m]].win++;
}

// one batched verify pass over the listed sequences' windows
void batch_verify_pass(lss_engine* e, const std::vector<int>& sq) {
  const auto& c = e->cfg;
  RowTok rt{};
  BatchSeqs bs{};
  bs.n = (int)sq.size();
  e->pass.clear();
  int M = 0;
  for (int i = 0; i < bs.n; ++i) {
    const SeqState& st = e->seqs[sq[i]];
    bs.seq[i] = sq[i];
    bs.row0[i] = M;
    bs.k[i] = st.win;
    e->pass.push_back(PassSeq{sq[i], M, st.win + 1, st.p});
    for (int j = 0; j <= st.win; ++j) rt.off[M + j] = sq[i] * kTokSlots + j;
    M += st.win + 1;
  }
  embed_rows(e, rt, M, hs_row(e, 0, 0), next_gain(e, nullptr, -1));
  for (int l = 0; l < c.n_layers; ++l)
    layer_forward(e, l, M, hs_row(e, l, 0), e->xa, e->pa, hs_row(e, l + 1, 0), next_gain(e, nullptr, l), MODE_BATCH,
                  0, 0);
  HeadRes* bres = e->res_all + e->nseq;
  head(e, 0, M, 0, 0, false, bres);
  hipLaunchKernelGGL(k_accept_b, dim3(1), dim3(ATT_SEQ_MAX), 0, e->stream, (const HeadRes*)bres, bs, e->res_all,
                     e->tok_all, kTokSlots);
  hipLaunchKernelGGL(k_gather_target_b, dim3(c.n_layers + 1, bs.n), dim3(256), 0, e->stream, e->hs, c.max_rows,
                     c.d_model, (const HeadRes*)e->res_all, bs, e->target_all,
                     (size_t)(c.n_layers + 1) * c.d_model);
}

int sync_res_all(lss_engine* e) {
  HIPCHK(hipMemcpyAsync(e->hres_all, e->res_all, sizeof(HeadRes) * (e->nseq + 1), hipMemcpyDeviceToHost, e->stream));
  HIPCHK(hipStreamSynchronize(e->stream));
  if (e->ev_used) prof_resolve(e);
  return LSS_OK;
}

}  // namespace

int lss_batch_draft(lss_engine* e, int32_t n, const int32_t* seqs, const uint8_t* masks, int32_t quant,
                    const int32_t* k, float exit_tau, int32_t* tokens_out, int32_t* k_done) {
  if (!e) return LSS_EINVAL;
  const auto& c = e->cfg;
  const int L = c.n_layers;
  if (!seqs_valid(e, n, seqs)) return fail(e, LSS_EINVAL, "batch_draft: sequences must be distinct and in range");
  if (!masks || !k || quant < 0 || quant > 1)
    return fail(e, LSS_EINVAL, "batch_draft: bad arguments (quant 0 or 1; the W8A8 draft is single-row)");
  if (e->inv_t > 0.f) return fail(e, LSS_EINVAL, "batch_draft: batches are greedy; sampling is on");
  seq_save(e);
  const int win_cap = std::min(kWinMax, c.max_rows - 1);
  int any = 0;
  for (int i = 0; i < n; ++i) {
    const SeqState& st = e->seqs[seqs[i]];
    if (!st.have_seq || st.pending_accept || st.tree > 0)
      return fail(e, LSS_ESTATE, "batch_draft: every sequence needs a prefill, no pending accept, no tree window");
    if (k[i] < 0) return fail(e, LSS_EINVAL, "batch_draft: negative k");
    if (st.win + k[i] > win_cap) return fail(e, LSS_ECAPACITY, "batch_draft: window would exceed its capacity");
    if (st.p + st.win + k[i] + 1 > c.max_seq) return fail(e, LSS_ECAPACITY, "batch_draft: KV capacity exceeded");
    any += k[i];
  }
  if (any > 0 && !tokens_out) return fail(e, LSS_EINVAL, "batch_draft: null tokens_out");
  const GemvScope gv(e, true);
  std::vector<int> start(n), done(n, 0);
  std::vector<char> live(n);
  for (int i = 0; i < n; ++i) {
    start[i] = e->seqs[seqs[i]].win;
    live[i] = k[i] > 0;
  }
  // groups of identical masks, in order of first appearance
  std::vector<int> grp(n, -1);
  int ng = 0;
  for (int i = 0; i < n; ++i) {
    for (int j = 0; j < i && grp[i] < 0; ++j)
      if (!std::memcmp(masks + (size_t)i * L, masks + (size_t)j * L, L)) grp[i] = grp[j];
    if (grp[i] < 0) grp[i] = ng++;
  }
  const int per_pass = std::min(c.max_rows, ATT_SEQ_MAX);
  for (int g = 0; g < ng; ++g) {
    int gi = 0;
    while (grp[gi] != g) ++gi;
    const uint8_t* mask = masks + (size_t)gi * L;
    for (;;) {
      std::vector<int> rows;                            // indices into seqs[] still drafting
      for (int i = 0; i < n; ++i)
        if (grp[i] == g && live[i] && done[i] < k[i]) rows.push_back(i);
      if (rows.empty()) break;
      for (size_t r0 = 0; r0 < rows.size(); r0 += per_pass) {
        std::vector<int> sq;
        for (size_t r = r0; r < std::min(rows.size(), r0 + per_pass); ++r) sq.push_back(seqs[rows[r]]);
        batch_draft_step(e, sq, mask, quant);
        if (exit_tau > 0.f) {
          int rc = check_launch(e, "batch_draft");
          if (rc) { seq_load(e, e->cur); return rc; }
          rc = sync_res_all(e);
          if (rc) { seq_load(e, e->cur); return rc; }
          const HeadRes& b = e->hres_all[e->nseq];
          for (size_t m = 0; m < sq.size(); ++m)
            if (b.pmax[m] < exit_tau) live[rows[r0 + m]] = 0;
        }
      }
      for (int i : rows) done[i]++;
    }
  }
  int rc = check_launch(e, "batch_draft");
  if (rc == LSS_OK && any > 0) rc = sync_res_all(e);
  if (rc == LSS_OK && any > 0)
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < done[i]; ++j)
        tokens_out[(size_t)i * LSS_WINDOW_MAX + j] = e->hres_all[seqs[i]].argmax[start[i] + j];
  if (k_done)
    for (int i = 0; i < n; ++i) k_done[i] = done[i];
  seq_load(e, e->cur);
  return rc;
}

int lss_batch_verify(lss_engine* e, int32_t n, const int32_t* seqs) {
  if (!e) return LSS_EINVAL;
  const auto& c = e->cfg;
  if (!seqs_valid(e, n, seqs)) return fail(e, LSS_EINVAL, "batch_verify: sequences must be distinct and in range");
  if (e->inv_t > 0.f) return fail(e, LSS_EINVAL, "batch_verify: batches are greedy; sampling is on");
  seq_save(e);
  for (int i = 0; i < n; ++i) {
    const SeqState& st = e->seqs[seqs[i]];
    if (!st.have_seq || st.pending_accept || st.tree > 0)
      return fail(e, LSS_ESTATE, "batch_verify: every sequence needs a prefill, no pending accept, no tree window");
    if (st.p + st.win + 1 > c.max_seq) return fail(e, LSS_ECAPACITY, "batch_verify: KV capacity exceeded");
  }
  const GemvScope gv(e);
  // passes: sequences in order while their rows fit max_rows and the pass
  // holds at most LSS_BATCH_PASS_SEQS sequences
  std::vector<int> sq;
  int rows = 0;
  for (int i = 0; i <= n; ++i) {
    const int r = i < n ? e->seqs[seqs[i]].win + 1 : 0;
    if (i == n || rows + r > c.max_rows || (int)sq.size() == LSS_BATCH_PASS_SEQS) {
      batch_verify_pass(e, sq);
      sq.clear();
      rows = 0;
    }
    if (i < n) {
      sq.push_back(seqs[i]);
      rows += r;
    }
  }
  const int rc = check_launch(e, "batch_verify");
  if (rc == LSS_OK)
    for (int i = 0; i < n; ++i) {
      SeqState& st = e->seqs[seqs[i]];
      st.verify_rows = st.win + 1;
      st.pending_accept = true;
    }
  seq_load(e, e->cur);
  return rc;
}

int lss_batch_accept(lss_engine* e, int32_t n, const int32_t* seqs, int32_t* n_accepted, int32_t* bonus,
                     int32_t* accepted_out) {
  if (!e) return LSS_EINVAL;
  if (!seqs_valid(e, n, seqs)) return fail(e, LSS_EINVAL, "batch_accept: sequences must be distinct and in range");
  seq_save(e);
  for (int i = 0; i < n; ++i)
    if (!e->seqs[seqs[i]].pending_accept) return fail(e, LSS_ESTATE, "batch_accept: a sequence has no verify pending");
  int rc = sync_res_all(e);
  if (rc) return rc;
  for (int i = 0; i < n; ++i) {
    SeqState& st = e->seqs[seqs[i]];
    const HeadRes& h = e->hres_all[seqs[i]];
    const int na = h.n;
    if (n_accepted) n_accepted[i] = na;
    if (bonus) bonus[i] = h.bonus;
    if (accepted_out)
      for (int j = 0; j <= na; ++j) accepted_out[(size_t)i * (LSS_WINDOW_MAX + 1) + j] = h.emit[j];
    st.target_pos = st.p + na;
    st.have_target = true;
    st.p += na + 1;
    st.win = 0;
    st.tree = 0;
    st.tree_D = 1;
    std::fill(st.valid.begin(), st.valid.end(), 0u);
    st.pending_accept = false;
  }
  seq_load(e, e->cur);
  return LSS_OK;
}

// ---------------------------------------------------------------- generation loop
int lss_generate(lss_engine* e, const int32_t* prompt, int32_t n_prompt, int32_t n_gen, const lss_policy* pol,
                 int32_t* out, lss_stats* stats) {
  if (!e) return LSS_EINVAL;
  const auto& c = e->cfg;
  const int L = c.n_layers;
  if (!pol || !out || n_gen < 1) return fail(e, LSS_EINVAL, "generate: bad arguments");
  if (pol->mode < LSS_MODE_AR || pol->mode > LSS_MODE_CASCADE) return fail(e, LSS_EINVAL, "generate: bad mode");
  if (pol->mode != LSS_MODE_AR && (pol->k_max < 0 || pol->k_max > std::min(kWinMax, c.max_rows - 1)))
    return fail(e, LSS_EINVAL, "generate: k_max out of range");
  if (pol->mode == LSS_MODE_STATIC && !pol->static_mask) return fail(e, LSS_EINVAL, "generate: static mask missing");
  if (pol->tree_width < 0 || pol->tree_width > TOPB_MAX || (pol->tree_width > 0 && pol->mode == LSS_MODE_AR))
    return fail(e, LSS_EINVAL, "generate: tree_width must be 0..8 and needs the static, DP or cascade mode");
  const int tree_depth = std::max(1, pol->tree_depth);   // 0: depth 1
  if (pol->tree_width > 0 && pol->mode != LSS_MODE_CASCADE &&
      (pol->tree_depth < 0 || (long)pol->tree_width * tree_depth > LSS_TREE_NODES_MAX))
    return fail(e, LSS_EINVAL, "generate: tree_depth must be >= 0 with tree_width * tree_depth <= 15");
  bool row_cost_set = false;
  for (int r = 0; r <= LSS_TREE_NODES_MAX; ++r) row_cost_set |= pol->row_cost[r] != 0.0;
  for (int r = 0; row_cost_set && r <= LSS_TREE_NODES_MAX; ++r)
    if (!(pol->row_cost[r] > 0.0)) return fail(e, LSS_EINVAL, "generate: row_cost entries must all be > 0 (or all 0)");
  if ((pol->mode == LSS_MODE_DP || pol->mode == LSS_MODE_CASCADE) && pol->interval < 1)
    return fail(e, LSS_EINVAL, "generate: interval < 1");
  if (pol->mode == LSS_MODE_CASCADE) {
    if (pol->n_levels < 1 || pol->n_levels > LSS_LEVELS_MAX) return fail(e, LSS_EINVAL, "generate: n_levels");
    for (int v = 0; v < pol->n_levels; ++v)
      if (pol->level_exit[v] < 0 || pol->level_exit[v] > pol->level_skip[v] || pol->level_skip[v] > L)
        return fail(e, LSS_EINVAL, "generate: level skip / exit out of range");
  }
  if ((long)n_prompt + n_gen + std::min(kWinMax, c.max_rows - 1) + 1 > c.max_seq)
    return fail(e, LSS_ECAPACITY, "generate: prompt + generation + window exceeds max_seq");
  const int rc_stop = check_stop(e, pol, "generate");
  if (rc_stop) return rc_stop;
  lss_stats st{};
  int32_t t0 = 0;
  int rc = lss_prefill(e, prompt, n_prompt, &t0);
  if (rc) return rc;
  int emitted = 0;
  out[emitted++] = t0;
  bool stopped = is_stop(pol, t0);
  const int nlev = pol->mode == LSS_MODE_CASCADE ? pol->n_levels : 1;
  std::vector<std::vector<uint8_t>> masks(nlev, std::vector<uint8_t>(L, 0));
  auto select = [&]() -> int {
    if (pol->mode == LSS_MODE_STATIC) {
      std::copy(pol->static_mask, pol->static_mask + L, masks[0].begin());
    } else if (pol->mode == LSS_MODE_DP) {
      int r = lss_select_layers_dp(e, pol->n_skip, masks[0].data(), nullptr);
      if (r) return r;
      st.dp_runs++;
    } else if (pol->mode == LSS_MODE_CASCADE) {
      for (int v = 0; v < nlev; ++v) {
        int r = lss_select_layers_dp_exit(e, pol->level_skip[v] - pol->level_exit[v], L - pol->level_exit[v],
                                     masks[v].data(), nullptr);
        if (r) return r;
        st.dp_runs++;
      }
    }
    return LSS_OK;
  };
  if (pol->mode != LSS_MODE_AR && !stopped) {
    rc = select();
    if (rc) return rc;
  }
  std::vector<double> acc_rate(nlev, router::kAInit);
  std::vector<int32_t> slot_levels;
  std::vector<int32_t> toks(64), acc(64);
  while (emitted < n_gen && !stopped) {
    const int budget = n_gen - emitted - 1;
    slot_levels.clear();
    if ((pol->mode == LSS_MODE_STATIC || pol->mode == LSS_MODE_DP) && pol->tree_width > 0) {
      if (budget > 0) {
        rc = lss_draft_tree(e, masks[0].data(), pol->quant, pol->tree_width, std::min(tree_depth, budget),
                            toks.data());
        if (rc) return rc;
      }
    } else if (pol->mode == LSS_MODE_STATIC || pol->mode == LSS_MODE_DP) {
      const int k = std::min(pol->k_max, budget);
      if (k > 0) {
        int kd = 0;
        rc = lss_draft(e, masks[0].data(), pol->quant, k, pol->exit_tau, toks.data(), &kd);
        if (rc) return rc;
      }
    } else if (pol->mode == LSS_MODE_CASCADE && pol->tree_width > 0) {
      // the levels routed into a token tree: width and k per level from the
      // tree router, depths drafted precise level first
      std::vector<double> t_hat(nlev);
      for (int v = 0; v < nlev; ++v) {
        int depth = 0;
        for (int l = 0; l < L; ++l) depth += masks[v][l] ? 0 : 1;
        t_hat[v] = router::predict(pol->beta, e->p, depth);
      }
      const double t_ver = router::predict(pol->beta, e->p, L);
      std::vector<int32_t> plan(nlev);
      int32_t B = 1;
      router::plan_tree(acc_rate.data(), t_hat.data(), nlev, t_ver, row_cost_set ? pol->row_cost : nullptr,
                        pol->k_max, pol->tree_width, std::min(LSS_TREE_NODES_MAX, c.max_rows - 1), &B, plan.data());
      for (int v = nlev - 1; v >= 0; --v)
        for (int i = 0; i < plan[v] && (int)slot_levels.size() < budget; ++i) slot_levels.push_back(v);
      const int D = (int)slot_levels.size();
      int branch = -1;
      if (D > 0) {
        std::vector<uint8_t> dm((size_t)D * L);
        std::vector<int32_t> dq(D);
        for (int j = 0; j < D; ++j) {
          std::copy(masks[slot_levels[j]].begin(), masks[slot_levels[j]].end(), dm.begin() + (size_t)j * L);
          dq[j] = pol->level_quant[slot_levels[j]];
        }
        rc = lss_draft_tree_levels(e, dm.data(), dq.data(), B, D, toks.data());
        if (rc) return rc;
      }
      const int k = e->win;
      rc = lss_verify(e, nullptr, k);
      if (rc) return rc;
      int n = 0, bonus = 0;
      rc = lss_accept_and_rollback(e, &n, &bonus, acc.data());
      if (rc) return rc;
      if (n > 0)                                        // the branch followed: its first node was emitted
        for (int b = 0; b < B; ++b)
          if (toks[(size_t)b * D] == acc[0]) branch = b;
      for (int i = 0; i <= n && emitted < n_gen && !stopped; ++i) {
        out[emitted++] = acc[i];
        stopped = is_stop(pol, acc[i]);
      }
      st.rounds++;
      st.drafted += k;
      st.accepted += n;
      router::update_tree(acc_rate.data(), nlev, slot_levels.data(), D, n, branch);
      if (!stopped && st.rounds % pol->interval == 0) {
        rc = select();
        if (rc) return rc;
      }
      continue;
    } else if (pol->mode == LSS_MODE_CASCADE) {
      std::vector<double> t_hat(nlev);
      for (int v = 0; v < nlev; ++v) {
        int depth = 0;
        for (int l = 0; l < L; ++l) depth += masks[v][l] ? 0 : 1;
        t_hat[v] = router::predict(pol->beta, e->p, depth);
      }
      const double t_ver = router::predict(pol->beta, e->p, L);
      std::vector<int32_t> plan(nlev);
      router::plan(acc_rate.data(), t_hat.data(), nlev, t_ver, pol->k_max, plan.data());
      int used = 0;
      for (int v = nlev - 1; v >= 0; --v) {
        const int k = std::min(plan[v], budget - used);
        if (k <= 0) continue;
        int kd = 0;
        rc = lss_draft(e, masks[v].data(), pol->level_quant[v], k, 0.f, toks.data(), &kd);
        if (rc) return rc;
        for (int i = 0; i < kd; ++i) slot_levels.push_back(v);
        used += kd;
      }
    }
    const int k = e->win;
    rc = lss_verify(e, nullptr, k);
    if (rc) return rc;
    int n = 0, bonus = 0;
    rc = lss_accept_and_rollback(e, &n, &bonus, acc.data());
    if (rc) return rc;
    for (int i = 0; i <= n && emitted < n_gen && !stopped; ++i) {
      out[emitted++] = acc[i];
      stopped = is_stop(pol, acc[i]);
    }
    st.rounds++;
    st.drafted += k;
    st.accepted += n;
    if (pol->mode == LSS_MODE_CASCADE)
      router::update(acc_rate.data(), nlev, slot_levels.data(), (int)slot_levels.size(), n);
    if (!stopped && (pol->mode == LSS_MODE_DP || pol->mode == LSS_MODE_CASCADE) && st.rounds % pol->interval == 0) {
      rc = select();
      if (rc) return rc;
    }
  }
  st.emitted = emitted;
  if (stats) *stats = st;
  return LSS_OK;
}

int lss_generate_batch(lss_engine* e, int32_t n, const int32_t* prompts, const int32_t* lens, int32_t n_gen,
                       const lss_policy* pol, int32_t* out, lss_stats* stats) {
  if (!e) return LSS_EINVAL;
  const auto& c = e->cfg;
  const int L = c.n_layers;
  if (!pol || !out || !prompts || !lens || n_gen < 1 || n < 1 || n > e->nseq)
    return fail(e, LSS_EINVAL, "generate_batch: bad arguments (1 <= n_seqs <= max_seqs)");
  if (pol->mode != LSS_MODE_AR && pol->mode != LSS_MODE_STATIC && pol->mode != LSS_MODE_DP)
    return fail(e, LSS_EINVAL, "generate_batch: modes AR, STATIC and DP only");
  if (pol->tree_width > 0 || pol->quant < 0 || pol->quant > 1 || e->inv_t > 0.f)
    return fail(e, LSS_EINVAL, "generate_batch: no trees, no W8A8 draft, greedy only");
  if (pol->mode != LSS_MODE_AR && (pol->k_max < 0 || pol->k_max > std::min(kWinMax, c.max_rows - 1)))
    return fail(e, LSS_EINVAL, "generate_batch: k_max out of range");
  if (pol->mode == LSS_MODE_STATIC && !pol->static_mask) return fail(e, LSS_EINVAL, "generate_batch: static mask missing");
  if (pol->mode == LSS_MODE_DP && pol->interval < 1) return fail(e, LSS_EINVAL, "generate_batch: interval < 1");
  for (int i = 0; i < n; ++i)
    if (lens[i] < 1 || (long)lens[i] + n_gen + std::min(kWinMax, c.max_rows - 1) + 1 > c.max_seq)
      return fail(e, LSS_ECAPACITY, "generate_batch: a prompt is empty or prompt + generation + window exceeds max_seq");
  const int rc_stop = check_stop(e, pol, "generate_batch");
  if (rc_stop) return rc_stop;
  const int cur0 = e->cur;
  std::vector<int32_t> seqs(n);
  std::vector<uint8_t> masks((size_t)n * L, 0);
  std::vector<int> emitted(n, 0);
  std::vector<uint8_t> stopped(n, 0);
  std::vector<lss_stats> st(n);
  int rc = LSS_OK;
  auto fin = [&](int r) {
    if (e->cur != cur0) {
      seq_save(e);
      seq_load(e, cur0);
    }
    return r;
  };
  auto dp = [&](int i) -> int {
    int r = lss_seq_select(e, i);
    if (r) return r;
    r = lss_select_layers_dp(e, pol->n_skip, masks.data() + (size_t)i * L, nullptr);
    if (r == LSS_OK) st[i].dp_runs++;
    return r;
  };
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    seqs[i] = i;
    rc = lss_seq_select(e, i);
    int32_t t0 = 0;
    if (rc == LSS_OK) rc = lss_prefill(e, prompts + off, lens[i], &t0);
    if (rc) return fin(rc);
    off += lens[i];
    out[(size_t)i * n_gen] = t0;
    emitted[i] = 1;
    stopped[i] = is_stop(pol, t0);
    if (pol->mode == LSS_MODE_STATIC) std::copy(pol->static_mask, pol->static_mask + L, masks.begin() + (size_t)i * L);
    if (pol->mode == LSS_MODE_DP && !stopped[i] && (rc = dp(i))) return fin(rc);
  }
  std::vector<int32_t> act, dk, done(n), toks((size_t)n * LSS_WINDOW_MAX), na(n), acc((size_t)n * (LSS_WINDOW_MAX + 1));
  std::vector<uint8_t> dmask;
  for (;;) {
    act.clear();
    for (int i = 0; i < n; ++i)
      if (emitted[i] < n_gen && !stopped[i]) act.push_back(i);
    if (act.empty()) break;
    const int na_ = (int)act.size();
    std::fill(done.begin(), done.end(), 0);
    if (pol->mode != LSS_MODE_AR) {
      dk.assign(na_, 0);
      dmask.assign((size_t)na_ * L, 0);
      for (int a = 0; a < na_; ++a) {
        dk[a] = std::min(pol->k_max, n_gen - emitted[act[a]] - 1);
        std::copy(masks.begin() + (size_t)act[a] * L, masks.begin() + (size_t)(act[a] + 1) * L,
                  dmask.begin() + (size_t)a * L);
      }
      rc = lss_batch_draft(e, na_, act.data(), dmask.data(), pol->quant, dk.data(), pol->exit_tau, toks.data(),
                           done.data());
      if (rc) return fin(rc);
    }
    rc = lss_batch_verify(e, na_, act.data());
    if (rc == LSS_OK) rc = lss_batch_accept(e, na_, act.data(), na.data(), nullptr, acc.data());
    if (rc) return fin(rc);
    for (int a = 0; a < na_; ++a) {
      const int i = act[a];
      for (int j = 0; j <= na[a] && emitted[i] < n_gen && !stopped[i]; ++j) {
        const int32_t tk = acc[(size_t)a * (LSS_WINDOW_MAX + 1) + j];
        out[(size_t)i * n_gen + emitted[i]++] = tk;
        stopped[i] = is_stop(pol, tk);
      }
      st[i].rounds++;
      st[i].drafted += done[a];
      st[i].accepted += na[a];
      if (!stopped[i] && pol->mode == LSS_MODE_DP && st[i].rounds % pol->interval == 0 && (rc = dp(i)))
        return fin(rc);
    }
  }
  for (int i = 0; i < n; ++i) {
    st[i].emitted = emitted[i];
    if (stats) stats[i] = st[i];
  }
  return fin(LSS_OK);
}

int lss_profile_kernel(lss_engine* e, int32_t epi, int32_t rows, int32_t enable) {
  if (!e) return LSS_EINVAL;
  if (enable && (epi < 0 || (epi > 3 && (epi < 16 || epi > 18)) || rows < 0))
    return fail(e, LSS_EINVAL, "profile_kernel: bad epilogue / rows");
  HIPCHK(hipStreamSynchronize(e->stream));
  prof_resolve(e);
  if (!enable) {
    e->prof_epi = -1;
    return LSS_OK;
  }
  if (e->ev_start.empty()) {
    const int n = 2048;
    e->ev_start.resize(n);
    e->ev_stop.resize(n);
    for (int i = 0; i < n; ++i) {
      HIPCHK(hipEventCreate(&e->ev_start[i]));
      HIPCHK(hipEventCreate(&e->ev_stop[i]));
    }
  }
  e->prof_epi = epi;
  e->prof_rows = rows;
  e->prof_ms = 0.0;
  e->prof_launches = 0;
  e->prof_bytes = 0;
  return LSS_OK;
}

int lss_profile_read(lss_engine* e, double* total_ms, int64_t* launches, int64_t* bytes) {
  if (!e) return LSS_EINVAL;
  HIPCHK(hipStreamSynchronize(e->stream));
  prof_resolve(e);
  if (total_ms) *total_ms = e->prof_ms;
  if (launches) *launches = e->prof_launches;
  if (bytes) *bytes = e->prof_bytes;
  return LSS_OK;
}

// ---------------------------------------------------------------- router ABI
int lss_router_plan(const double* a, const double* t_hat, int32_t n_levels, double t_verify, int32_t k_max,
                    int32_t* plan_out) {
  if (!a || !t_hat || !plan_out || n_levels < 1 || n_levels > LSS_LEVELS_MAX || k_max < 0 || k_max > kWinMax)
    return LSS_EINVAL;
  router::plan(a, t_hat, n_levels, t_verify, k_max, plan_out);
  return LSS_OK;
}

int lss_router_update(double* a, int32_t n_levels, const int32_t* slot_levels, int32_t k, int32_t n) {
  if (!a || n_levels < 1 || n_levels > LSS_LEVELS_MAX || k < 0 || n < 0 || n > k || (k > 0 && !slot_levels))
    return LSS_EINVAL;
  for (int i = 0; i < k; ++i)
    if (slot_levels[i] < 0 || slot_levels[i] >= n_levels) return LSS_EINVAL;
  router::update(a, n_levels, slot_levels, k, n);
  return LSS_OK;
}

int lss_router_plan_tree(const double* a, const double* t_hat, int32_t n_levels, double t_verify,
                         const double* row_cost, int32_t k_max, int32_t b_max, int32_t nodes_max,
                         int32_t* width_out, int32_t* plan_out) {
  if (!a || !t_hat || !plan_out || !width_out || n_levels < 1 || n_levels > LSS_LEVELS_MAX || k_max < 0 ||
      k_max > kWinMax || b_max < 1 || b_max > TOPB_MAX || nodes_max < 1 || nodes_max > LSS_TREE_NODES_MAX)
    return LSS_EINVAL;
  router::plan_tree(a, t_hat, n_levels, t_verify, row_cost, k_max, b_max, nodes_max, width_out, plan_out);
  return LSS_OK;
}

int lss_router_update_tree(double* a, int32_t n_levels, const int32_t* depth_levels, int32_t D, int32_t n,
                           int32_t branch) {
  if (!a || n_levels < 1 || n_levels > LSS_LEVELS_MAX || D < 0 || n < 0 || n > D || (D > 0 && !depth_levels) ||
      branch < -1 || branch >= TOPB_MAX || (n > 0) != (branch >= 0))
    return LSS_EINVAL;
  for (int i = 0; i < D; ++i)
    if (depth_levels[i] < 0 || depth_levels[i] >= n_levels) return LSS_EINVAL;
  router::update_tree(a, n_levels, depth_levels, D, n, branch);
  return LSS_OK;
}

int lss_latency_fit(const double* samples, int32_t n, double* beta_out) {
  if (!samples || !beta_out || n < 3) return LSS_EINVAL;
  return router::fit(samples, n, beta_out) ? LSS_OK : LSS_EINVAL;
}

}  // extern "C"
