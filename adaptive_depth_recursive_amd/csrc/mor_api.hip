// Host runtime behind include/mor.h: config validation, workspace plan, weight packing, the
// enqueue order of the MoR prefill and of a depth-wise batched decode iteration (replayed from a
// captured graph). Host code only; every step of the computation runs in the kernels of
// k_gemm_bf16.hip / k_gemm.hip, k_attn_bf16.hip / k_attn.hip, k_route.hip and k_decode.hip.
//
// Prefill order (MoR paper A.1-A.3; reading notes 1, 2.1-2.2, 3.1-3.2):
//   first layer on all tokens -> router r=1
//   for r = 1..N_r: select the active set, gather its rows, run the n_s shared layers on them
//                   (attention over the tokens active at r, or over the recursion-1 tokens under
//                   KV sharing), gated scatter back into H fused with the router of r+1
//   last layer on all tokens.
// Expert-choice counts are static, so nothing is read back to the host during a call.
#include <climits>
#include <mutex>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "mor.h"
#include "mor_internal.h"

using namespace mor;

namespace {

thread_local std::string g_err;

mor_status fail(mor_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define HIPCHK(expr)                                                              \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess)                                                         \
      return fail(MOR_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));  \
  } while (0)

struct BlockPacked {
  void* wqkv;   // [(Hq + 2 Hkv) hd][d]: Wq rows, then Wk, then Wv
  void* wo;     // [d][Hq hd]
  void* wgu;    // [2 d_ff][d]: gate/up rows in alternating groups of 16
  void* wd;     // [d][d_ff]
  float* g_attn;
  float* g_ffn;
};

constexpr size_t kAlign = 256;

// K splits of the decode projections: enough workgroups to spread the weight streaming over the
// CUs (a projection has only N/16 column groups of 64 slot rows). Their consumers fold the
// partial sums in split order (decode attention folds at most kMaxQkvSplits of the QKV
// projection, the row kernels at most 8 of the residual ones). QKV 2, O 4, down 4 measured best
// at the 360M shape (QKV 4: 0.6% slower per iteration; O 2: 1.8%; down 2: 11%).
#ifndef MOR_DEC_SPLIT_QKV
#define MOR_DEC_SPLIT_QKV 2
#endif
#ifndef MOR_DEC_SPLIT_O
#define MOR_DEC_SPLIT_O 4
#endif
#ifndef MOR_DEC_SPLIT_DOWN
#define MOR_DEC_SPLIT_DOWN 4
#endif
constexpr int kSplitQKV = MOR_DEC_SPLIT_QKV, kSplitO = MOR_DEC_SPLIT_O, kSplitDown = MOR_DEC_SPLIT_DOWN;
constexpr int kSplitPx = kSplitO > kSplitDown ? kSplitO : kSplitDown;
static_assert(kSplitQKV >= 1 && kSplitQKV <= kMaxQkvSplits, "QKV split out of range");
static_assert(kSplitO >= 1 && kSplitO <= 8 && kSplitDown >= 1 && kSplitDown <= 8, "split out of range");

struct Cursor {
  char* base;
  size_t off = 0;
  template <typename P>
  P* take(size_t bytes) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

}  // namespace

// Scratch of mor_route_noalloc: the set's row offsets [MOR_NOALLOC_MAX_BATCH + 1] and row map
// [MOR_NOALLOC_MAX_TOKENS]. One copy per GPU, held until the process ends; its device address is
// looked up once per device (scratch_on) and only that address is handed to kernels.
constexpr int kNoallocInts = MOR_NOALLOC_MAX_BATCH + 1 + MOR_NOALLOC_MAX_TOKENS;
static __device__ __align__(256) int scratch[kNoallocInts];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static int* g_scratch_ptr[kMaxDevices] = {};

struct mor_handle_s {
  mor_config cfg;
  int device = 0;                // the GPU current at mor_init (the handle's workspace lives there)
  int n_s = 0, es = 0, nq = 0, nkv = 0, nqkv = 0, kpad = 0, nstreams = 0;
  size_t MT = 0;                 // max_batch * max_seq
  std::vector<BlockPacked> blk;  // 0 = first, 1..n_s = shared, n_s + 1 = last
  float* router_w = nullptr;
  float* router_b = nullptr;
  bool has_bias = false;
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;
  float* X = nullptr;
  void* Xn = nullptr;
  void* Q = nullptr;
  void* O = nullptr;
  void* Hf = nullptr;
  char* kv = nullptr;
  size_t kv_half_bytes = 0;      // bytes of K (= bytes of V^T) of one stream
  int* act = nullptr;            // [N_r + 1][MT]   set r as [B][T] (positions, -1 padded)
  int* cnt = nullptr;            // [N_r + 1][max_batch]
  int* meta = nullptr;           // [N_r + 2][max_batch + 1]; the last slot is scratch
  float* z = nullptr;            // [N_r + 1][MT]   z[r] by source row b*T + pos
  float* tc_logits = nullptr;    // [N_r][MT]
  int* depth = nullptr;          // [MT]
  float* prob = nullptr;         // [MT]
  int* rows_all = nullptr;       // 4 x [MT]: pos, src, seq, idx of the all-token set
  int* rows = nullptr;           // 4 x [MT]: the same for the current active set
  float* gate = nullptr;         // [MT]
  unsigned* err = nullptr;
  unsigned long long* clk = nullptr;  // [2] shader cycles / real-time ticks of the timed projection kind
  // depth-wise batched decode
  bool decode = false;
  int kv_pages = 0, pps = 0, LS = 0;
  size_t page_bytes = 0;
  DecArgs dec{};
  int* dreq_len = nullptr;       // [max_requests]
  int* dreq_off = nullptr;       // [max_requests]
  void* dXn = nullptr;           // [64][d]
  float* dQkv = nullptr;         // [kSplitQKV][64][nqkv] partial sums
  float* dPx = nullptr;          // [kSplitPx][64][d] partial sums of the O / down projections
  void* dO = nullptr;            // [64][nq]
  void* dHf = nullptr;           // [64][d_ff]
  bool submitted = false;
  int last_B = 0, last_T = 0;    // shape of the last mor_prefill (the prefix a decode can continue)
  // decode iterations replayed as a captured HIP graph (kernel arguments fixed per submission)
  hipStream_t cap_stream = nullptr;
  hipGraph_t dec_graph = nullptr;
  hipGraphExec_t dec_exec = nullptr;
  // measurement: HIP events around every launch of one kernel kind
  int timing_kind = 0;
  std::vector<hipEvent_t> ev;
  size_t ev_used = 0;
  hipStream_t ev_stream = nullptr;
};

namespace {

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Sharing scheme helpers (mor_sharing). Under MIDDLE_* sharing the first and last layers are
// unique and the N_r recursions share the L-2 layers between them; otherwise all L are shared.
bool middle_sharing(const mor_config& c) {
  return c.sharing == MOR_SHARE_MIDDLE_CYCLE || c.sharing == MOR_SHARE_MIDDLE_SEQUENCE;
}
int shared_per_rec(const mor_config& c) {
  return (middle_sharing(c) ? c.n_layers - 2 : c.n_layers) / c.n_rec;
}
// Shared block (1..n_s) of position j (1..n_s) of recursion r (1..N_r): the cycle schemes reuse
// block j at every recursion; the sequence schemes repeat each block on N_r consecutive layers.
int block_of(const mor_config& c, int n_s, int r, int j) {
  if (c.sharing == MOR_SHARE_MIDDLE_CYCLE || c.sharing == MOR_SHARE_CYCLE) return j;
  const int u = (r - 1) * n_s + (j - 1);
  return u / c.n_rec + 1;
}

mor_status validate(const mor_config* c) {
  if (!c) return fail(MOR_E_INVALID, "null config");
  if (c->dtype != MOR_F32 && c->dtype != MOR_BF16) return fail(MOR_E_INVALID, "dtype");
  if (c->routing < 0 || c->routing > 2) return fail(MOR_E_INVALID, "routing");
  if (c->kv_mode < 0 || c->kv_mode > 1) return fail(MOR_E_INVALID, "kv_mode");
  if (c->gate_mode < 0 || c->gate_mode > 1) return fail(MOR_E_INVALID, "gate_mode");
  if (c->sharing < 0 || c->sharing > 3) return fail(MOR_E_INVALID, "sharing");
  if (c->d_model <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->d_ff <= 0 || c->n_rec < 1 || c->n_rec > MOR_MAX_REC)
    return fail(MOR_E_INVALID, "non-positive dimension or n_rec outside 1..8");
  const int span = middle_sharing(*c) ? c->n_layers - 2 : c->n_layers;
  if (span < c->n_rec || span % c->n_rec)
    return fail(MOR_E_INVALID, middle_sharing(*c) ? "n_layers - 2 must be a positive multiple of n_rec"
                                                  : "n_layers must be a positive multiple of n_rec");
  const int n_s = span / c->n_rec;
  if (n_s > MOR_MAX_SHARED) return fail(MOR_E_SHAPE, "more than 64 shared layers");
  if (c->d_model % 64 || c->d_ff % 64) return fail(MOR_E_SHAPE, "d_model and d_ff must be multiples of 64");
  if (c->dtype == MOR_BF16 && c->head_dim != 64) return fail(MOR_E_SHAPE, "bf16 needs head_dim 64");
  if (c->dtype == MOR_F32 && c->head_dim != 16 && c->head_dim != 32 && c->head_dim != 64)
    return fail(MOR_E_SHAPE, "fp32 needs head_dim 16, 32 or 64");
  if (c->n_q_heads % c->n_kv_heads || c->n_q_heads / c->n_kv_heads > 4)
    return fail(MOR_E_SHAPE, "n_q_heads must be 1..4 times n_kv_heads");
  if ((c->n_q_heads * c->head_dim) % 64) return fail(MOR_E_SHAPE, "n_q_heads * head_dim % 64 != 0");
  if (c->cap_den <= 0) return fail(MOR_E_INVALID, "cap_den");
  for (int r = 0; r < c->n_rec; ++r) {
    if (c->cap_num[r] < 0 || c->cap_num[r] > c->cap_den) return fail(MOR_E_INVALID, "capacity outside [0, 1]");
    if (r && c->cap_num[r] > c->cap_num[r - 1]) return fail(MOR_E_INVALID, "capacities must be non-increasing");
  }
  if (c->max_batch < 1 || c->max_seq < 1 || c->max_seq > 8192)
    return fail(MOR_E_SHAPE, "max_batch >= 1 and 1 <= max_seq <= 8192");
  if ((double)c->max_batch * c->max_seq * (double)std::max(c->d_ff, c->d_model) > 2.0e9)
    return fail(MOR_E_SHAPE, "max_batch * max_seq too large");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return fail(MOR_E_INVALID, "rms_eps / rope_theta");
  if (c->max_slots < 0 || c->max_slots > 64) return fail(MOR_E_SHAPE, "max_slots must be 0..64");
  if (c->max_slots > 0) {
    if (c->routing != MOR_ROUTE_THRESHOLD) return fail(MOR_E_INVALID, "decode needs threshold routing");
    if (c->sharing != MOR_SHARE_MIDDLE_CYCLE) return fail(MOR_E_INVALID, "decode needs middle-cycle sharing");
    const int P = c->kv_page_tokens;
    if (P != 16 && P != 32 && P != 64 && P != 128) return fail(MOR_E_SHAPE, "kv_page_tokens must be 16, 32, 64 or 128");
    if (c->kv_pages < 0 || c->max_requests < 1) return fail(MOR_E_INVALID, "kv_pages >= 0, max_requests >= 1");
    if (c->d_model > 4096) return fail(MOR_E_SHAPE, "decode supports d_model up to 4096");
    if (((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim) % 32)
      return fail(MOR_E_SHAPE, "decode needs (n_q_heads + 2 n_kv_heads) * head_dim % 32 == 0");
  }
  return MOR_OK;
}

// Walks the workspace; with base == nullptr only sizes it.
size_t plan(const mor_config& c, mor_handle_s* h, char* base) {
  Cursor cur{base};
  const int n_s = shared_per_rec(c);
  const size_t es = c.dtype == MOR_BF16 ? 2 : 4;
  const size_t d = c.d_model, dff = c.d_ff, hd = c.head_dim;
  const size_t nq = c.n_q_heads * hd, nkv = c.n_kv_heads * hd, nqkv = nq + 2 * nkv;
  const size_t MT = (size_t)c.max_batch * c.max_seq;
  const int R = c.n_rec;
  const size_t kpad = (size_t)ceil_div(c.max_seq, 64) * 64;
  const int nstreams = 2 + R * n_s;
  std::vector<BlockPacked> blk(n_s + 2);
  for (auto& b : blk) {
    b.wqkv = cur.take<void>(nqkv * d * es);
    b.wo = cur.take<void>(d * nq * es);
    b.wgu = cur.take<void>(2 * dff * d * es);
    b.wd = cur.take<void>(d * dff * es);
    b.g_attn = cur.take<float>(d * 4);
    b.g_ffn = cur.take<float>(d * 4);
  }
  float* router_w = cur.take<float>(R * d * 4);
  float* router_b = cur.take<float>(R * 4);
  float* rope_cos = cur.take<float>((size_t)c.max_seq * (hd / 2) * 4);
  float* rope_sin = cur.take<float>((size_t)c.max_seq * (hd / 2) * 4);
  float* X = cur.take<float>(MT * d * 4);
  void* Xn = cur.take<void>(MT * d * es);
  void* Q = cur.take<void>(MT * nq * es);
  void* O = cur.take<void>(MT * nq * es);
  void* Hf = cur.take<void>(MT * dff * es);
  const size_t kv_half = (size_t)c.max_batch * kpad * nkv * es;
  char* kv = cur.take<char>(kv_half * 2 * nstreams);
  int* act = cur.take<int>((R + 1) * MT * 4);
  int* cnt = cur.take<int>((R + 1) * (size_t)c.max_batch * 4);
  int* meta = cur.take<int>((R + 2) * (size_t)(c.max_batch + 1) * 4);
  float* z = cur.take<float>((R + 1) * MT * 4);
  float* tc_logits = cur.take<float>(R * MT * 4);
  int* depth = cur.take<int>(MT * 4);
  float* prob = cur.take<float>(MT * 4);
  int* rows_all = cur.take<int>(4 * MT * 4);
  int* rows = cur.take<int>(4 * MT * 4);
  float* gate = cur.take<float>(MT * 4);
  unsigned* err = cur.take<unsigned>(64);
  unsigned long long* clk = cur.take<unsigned long long>(2 * 8);
  // decode engine
  const int S = c.max_slots;
  const int P = S ? c.kv_page_tokens : 1;
  const int pps = ceil_div(c.max_seq, P);
  const int LS = 2 + R * n_s;
  const size_t page_elems = 2 * nkv * (size_t)P;
  const size_t page_bytes = page_elems * es;
  const int kv_pages = S ? (c.kv_pages ? c.kv_pages : S * LS * pps) : 0;
  DecArgs da{};
  int *dreq_len = nullptr, *dreq_off = nullptr;
  void *dXn = nullptr, *dO = nullptr, *dHf = nullptr;
  float* dQkv = nullptr;
  float* dPx = nullptr;
  if (S) {
    da.sl_req = cur.take<int>(S * 4); da.sl_pos = cur.take<int>(S * 4);
    da.sl_base = cur.take<int>(S * 4);
    da.sl_depth = cur.take<int>(S * 4); da.sl_first = cur.take<int>(S * 4);
    da.sl_part = cur.take<int>(S * 4); da.sl_exit = cur.take<int>(S * 4);
    da.sl_cnt = cur.take<int>((size_t)S * R * 4);
    da.ptab = cur.take<int>((size_t)S * LS * pps * 4);
    da.free_pages = cur.take<int>((size_t)kv_pages * 4);
    da.glob = cur.take<int>(G_COUNT * 4);
    da.stats = cur.take<unsigned long long>(ST_COUNT * 8);
    dreq_len = cur.take<int>((size_t)c.max_requests * 4);
    dreq_off = cur.take<int>((size_t)c.max_requests * 4);
    da.X = cur.take<float>(64 * d * 4);
    da.Hs = cur.take<float>(64 * d * 4);
    da.gate = cur.take<float>(64 * 4);
    dXn = cur.take<void>(64 * d * es);
    dQkv = cur.take<float>((size_t)kSplitQKV * 64 * nqkv * 4);
    dPx = cur.take<float>((size_t)kSplitPx * 64 * d * 4);
    dO = cur.take<void>(64 * nq * es);
    dHf = cur.take<void>(64 * dff * es);
    da.pool = cur.take<void>((size_t)kv_pages * page_bytes);
  }
  if (h) {
    h->n_s = n_s; h->es = (int)es; h->nq = (int)nq; h->nkv = (int)nkv; h->nqkv = (int)nqkv;
    h->kpad = (int)kpad; h->nstreams = nstreams; h->MT = MT;
    h->blk = blk; h->router_w = router_w; h->router_b = router_b;
    h->rope_cos = rope_cos; h->rope_sin = rope_sin;
    h->X = X; h->Xn = Xn; h->Q = Q; h->O = O; h->Hf = Hf;
    h->kv = kv; h->kv_half_bytes = kv_half;
    h->act = act; h->cnt = cnt; h->meta = meta; h->z = z; h->tc_logits = tc_logits;
    h->depth = depth; h->prob = prob; h->rows_all = rows_all; h->rows = rows; h->gate = gate;
    h->err = err;
    h->clk = clk;
    h->decode = S > 0;
    if (S) {
      h->kv_pages = kv_pages; h->pps = pps; h->LS = LS; h->page_bytes = page_bytes;
      h->dreq_len = dreq_len; h->dreq_off = dreq_off;
      h->dXn = dXn; h->dQkv = dQkv; h->dPx = dPx; h->dO = dO; h->dHf = dHf;
      da.S = S; da.R = R; da.n_s = n_s; da.P = P; da.pps = pps; da.LS = LS;
      da.d = (int)d; da.hd = (int)hd; da.hkv = c.n_kv_heads; da.hq = c.n_q_heads;
      da.nq = (int)nq; da.nkv = (int)nkv; da.nqkv = (int)nqkv;
      da.kv_share = c.kv_mode == MOR_KV_SHARE_FIRST;
      da.unit_gate = c.gate_mode == MOR_GATE_UNIT;
      da.page_elems = (long long)page_elems;
      da.kv_pages = kv_pages;
      da.err = err;
      da.req_len = dreq_len; da.req_off = dreq_off;
      da.router_w = router_w; da.router_b = router_b;
      da.rope_cos = rope_cos; da.rope_sin = rope_sin;
      da.qkv = dQkv; da.kqkv = kSplitQKV; da.px = dPx; da.o = dO;
      da.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)hd));
      da.es = (int)es;
      da.layer_weight_bytes = (long long)((nqkv * d + d * nq + 2 * dff * d + d * dff) * es);
      h->dec = da;
    }
  }
  return cur.off + kAlign;
}

// ------------------------------------------------------------------ one decoder layer
struct RowSet {
  const int* meta;     // row-set descriptor
  const int* cnt;      // [B] rows per sequence
  const int* rows;     // 4 x [MT] pos/src/seq/idx
  int m_upper;         // grid bound on the row count
  int max_per_seq;     // grid bound on rows per sequence
  bool exact;          // m_upper is the row count itself (not only a bound known on the host)
};
struct KeySet {
  const void* k;
  const void* vt;
  const int* kpos;     // [B][T]
  const int* kcnt;     // [B]
};

enum { KIND_QKV = 1, KIND_ATTN = 2, KIND_O = 3, KIND_GATE_UP = 4, KIND_DOWN = 5, KIND_ROUTER = 6,
       KIND_SELECT = 7, KIND_GATHER = 8, KIND_SCATTER = 9, KIND_NORM = 10, KIND_LAST = KIND_NORM };

// Brackets one launch with a pair of events when this kind is being timed.
struct TimedLaunch {
  mor_handle_s* h;
  bool on;
  hipStream_t s;
  TimedLaunch(mor_handle_s* h_, int kind, hipStream_t s_)
      : h(h_), on(h_->timing_kind == kind && h_->ev_used + 2 <= h_->ev.size()), s(s_) {
    if (on) {
      (void)hipEventRecord(h->ev[h->ev_used], s);
      h->ev_stream = s;
    }
  }
  ~TimedLaunch() {
    if (on) {
      (void)hipEventRecord(h->ev[h->ev_used + 1], s);
      h->ev_used += 2;
    }
  }
};

// One Llama block on the rows of rs, updating X in place; with x_in, the block's input rows are
// read from x_in instead and X receives the output (every row of rs is written).
template <typename E>
mor_status run_layer(mor_handle_s* h, const BlockPacked& w, float* X, const RowSet& rs,
                     void* k_dst, void* vt_dst, const KeySet& keys, int B, int T, hipStream_t s,
                     const float* x_in = nullptr) {
  const mor_config& c = h->cfg;
  const int d = c.d_model, dff = c.d_ff, MT = (int)h->MT;
  E* Xn = reinterpret_cast<E*>(h->Xn);
  {
    TimedLaunch t(h, KIND_NORM, s);
    HIPCHK(launch_rmsnorm<E>(x_in ? x_in : X, d, rs.meta, rs.m_upper, w.g_attn, c.rms_eps, Xn, s));
  }

  GemmEpi ep{};
  ep.rows_bound = !rs.exact;
  ep.q = h->Q; ep.ldq = h->nq;
  ep.k = k_dst; ep.vt = vt_dst;
  ep.nq = h->nq; ep.nkv = h->nkv; ep.hd = c.head_dim; ep.hkv = c.n_kv_heads; ep.kpad = h->kpad;
  ep.rowpos = rs.rows; ep.rowseq = rs.rows + 2 * (size_t)MT; ep.rowidx = rs.rows + 3 * (size_t)MT;
  ep.rope_cos = h->rope_cos; ep.rope_sin = h->rope_sin;
  const int n_qkv = k_dst ? h->nqkv : h->nq;
  {
    TimedLaunch t(h, KIND_QKV, s);
    ep.clk = t.on ? h->clk : nullptr;
    HIPCHK(launch_gemm<E>(EPI_QKV, Xn, reinterpret_cast<const E*>(w.wqkv), n_qkv, d, rs.m_upper, rs.meta, ep, s));
  }

  AttnArgs aa{};
  aa.q = h->Q; aa.ldq = h->nq; aa.qmeta = rs.meta; aa.qcnt = rs.cnt; aa.qpos = rs.rows;
  aa.k = keys.k; aa.vt = keys.vt; aa.kpos = keys.kpos; aa.ldkpos = T; aa.kcnt = keys.kcnt;
  aa.kpad = h->kpad; aa.hkv = c.n_kv_heads; aa.hq = c.n_q_heads; aa.hd = c.head_dim;
  aa.o = h->O; aa.ldo = h->nq;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  {
    TimedLaunch t(h, KIND_ATTN, s);
    HIPCHK(launch_attention<E>(aa, B, rs.max_per_seq, s));
  }

  GemmEpi er{};
  er.rows_bound = !rs.exact;
  er.x = X; er.ldx = d;
  er.xin = x_in;
  {
    TimedLaunch t(h, KIND_O, s);
    er.clk = t.on ? h->clk : nullptr;
    HIPCHK(launch_gemm<E>(EPI_RESID, reinterpret_cast<const E*>(h->O), reinterpret_cast<const E*>(w.wo), d, h->nq, rs.m_upper, rs.meta, er, s));
  }
  er.xin = nullptr;
  {
    TimedLaunch t(h, KIND_NORM, s);
    HIPCHK(launch_rmsnorm<E>(X, d, rs.meta, rs.m_upper, w.g_ffn, c.rms_eps, Xn, s));
  }
  GemmEpi eg{};
  eg.rows_bound = !rs.exact;
  eg.h = h->Hf; eg.ldh = dff;
  {
    TimedLaunch t(h, KIND_GATE_UP, s);
    eg.clk = t.on ? h->clk : nullptr;
    HIPCHK(launch_gemm<E>(EPI_SWIGLU, Xn, reinterpret_cast<const E*>(w.wgu), 2 * dff, d, rs.m_upper, rs.meta, eg, s));
  }
  {
    TimedLaunch t(h, KIND_DOWN, s);
    er.clk = t.on ? h->clk : nullptr;
    HIPCHK(launch_gemm<E>(EPI_RESID, reinterpret_cast<const E*>(h->Hf), reinterpret_cast<const E*>(w.wd), d, dff, rs.m_upper, rs.meta, er, s));
  }
  return MOR_OK;
}

void* kv_k(mor_handle_s* h, int stream) { return h->kv + (size_t)stream * 2 * h->kv_half_bytes; }
void* kv_vt(mor_handle_s* h, int stream) { return h->kv + ((size_t)stream * 2 + 1) * h->kv_half_bytes; }

template <typename E>
mor_status prefill_impl(mor_handle_s* h, const float* h_in, int B, int T, float* H,
                        int32_t* sel_pos, int32_t* counts, float* logits, float* h_per_rec,
                        hipStream_t s) {
  const mor_config& c = h->cfg;
  const int R = c.n_rec, n_s = h->n_s, d = c.d_model;
  const size_t MT = h->MT, BT = (size_t)B * T;
  const size_t hbytes = BT * d * sizeof(float);
  int ks[MOR_MAX_REC];
  for (int r = 0; r < R; ++r) ks[r] = ceil_div((long)c.cap_num[r] * T, c.cap_den);

  const bool middle = middle_sharing(c);
  // with a unique first layer the input enters the stream through that layer (it reads h_in and
  // writes H); otherwise routing starts on a copy of the input
  if (H != h_in && !middle) HIPCHK(hipMemcpyAsync(H, h_in, hbytes, hipMemcpyDeviceToDevice, s));
  int* meta_r[MOR_MAX_REC + 2];
  for (int r = 0; r <= R + 1; ++r) meta_r[r] = h->meta + (size_t)r * (c.max_batch + 1);
  auto act_r = [&](int r) { return h->act + (size_t)r * MT; };
  auto cnt_r = [&](int r) { return h->cnt + (size_t)r * c.max_batch; };
  auto z_r = [&](int r) { return h->z + (size_t)r * MT; };
  HIPCHK(launch_init_sets(B, T, act_r(0), cnt_r(0), meta_r[0], h->rows_all, h->rows_all + MT,
                          h->rows_all + 2 * MT, h->rows_all + 3 * MT, s));
  if (logits && c.routing != MOR_ROUTE_TOKEN_CHOICE)
    HIPCHK(launch_fill_f32(h->z + MT, R * MT, NAN, s));

  const RowSet all{meta_r[0], cnt_r(0), h->rows_all, (int)BT, T, true};
  mor_status st = MOR_OK;
  if (middle) {
    const KeySet keys_first{kv_k(h, 0), kv_vt(h, 0), act_r(0), cnt_r(0)};
    st = run_layer<E>(h, h->blk[0], H, all, kv_k(h, 0), kv_vt(h, 0), keys_first, B, T, s,
                      H != h_in ? h_in : nullptr);
    if (st != MOR_OK) return st;
  }
  if (h_per_rec) HIPCHK(hipMemcpyAsync(h_per_rec, H, hbytes, hipMemcpyDeviceToDevice, s));

  const bool tc = c.routing == MOR_ROUTE_TOKEN_CHOICE;
  {
    TimedLaunch t(h, KIND_ROUTER, s);
    if (tc) {
      HIPCHK(launch_router_tc(H, d, (int)BT, h->router_w, R, h->tc_logits, h->depth, h->prob, s));
    } else {
      HIPCHK(launch_router(H, d, h->rows_all + MT, meta_r[0], (int)BT, h->router_w,
                           h->has_bias ? h->router_b : nullptr, z_r(1), s));
    }
  }
  const int sel_mode = c.routing == MOR_ROUTE_EC_TOPK ? SEL_EC
                       : c.routing == MOR_ROUTE_THRESHOLD ? SEL_THRESHOLD : SEL_TC;
  const int gate_kind = c.gate_mode == MOR_GATE_UNIT ? GATE_ASSIGN : tc ? GATE_TC : GATE_SIGMOID;
  for (int r = 1; r <= R; ++r) {
    {
      TimedLaunch t(h, KIND_SELECT, s);
      HIPCHK(launch_select(sel_mode, B, T, z_r(r), h->depth, act_r(r - 1), cnt_r(r - 1), ks[r - 1], r,
                           act_r(r), cnt_r(r), h->err, s));
    }
    HIPCHK(launch_offsets(cnt_r(r), B, meta_r[r], s));
    const int per_seq = sel_mode == SEL_EC ? std::min(ks[r - 1], T) : T;
    const int m_up = B * per_seq;
    {
      TimedLaunch t(h, KIND_GATHER, s);
      HIPCHK(launch_gather(H, d, act_r(r), meta_r[r], B, T, m_up, gate_kind, z_r(r), h->depth,
                           h->prob, r, h->X, h->rows, h->rows + MT, h->rows + 2 * MT, h->rows + 3 * MT,
                           h->gate, s));
    }
    // expert choice keeps exactly k_r tokens per sequence, and recursion 1 of the threshold and
    // token-choice routers runs every token; otherwise the count is known only on the device
    const RowSet rs{meta_r[r], cnt_r(r), h->rows, m_up, per_seq, sel_mode == SEL_EC || r == 1};
    for (int j = 1; j <= n_s; ++j) {
      const int sid = 1 + (r - 1) * n_s + (j - 1);
      const BlockPacked& wj = h->blk[block_of(c, n_s, r, j)];
      const bool share = c.kv_mode == MOR_KV_SHARE_FIRST && r >= 2;
      if (share) {
        const int s1 = 1 + (j - 1);
        const KeySet ks1{kv_k(h, s1), kv_vt(h, s1), act_r(1), cnt_r(1)};
        st = run_layer<E>(h, wj, h->X, rs, nullptr, nullptr, ks1, B, T, s);
      } else {
        const KeySet kr{kv_k(h, sid), kv_vt(h, sid), act_r(r), cnt_r(r)};
        st = run_layer<E>(h, wj, h->X, rs, kv_k(h, sid), kv_vt(h, sid), kr, B, T, s);
      }
      if (st != MOR_OK) return st;
    }
    const float* w_next = (!tc && r < R) ? h->router_w + (size_t)r * d : nullptr;
    const float* b_next = (w_next && h->has_bias) ? h->router_b + r : nullptr;
    {
      TimedLaunch t(h, KIND_SCATTER, s);
      HIPCHK(launch_scatter(H, h->X, d, meta_r[r], m_up, h->rows + MT, h->gate, w_next, b_next,
                            z_r(r + 1 <= R ? r + 1 : R), s));
    }
    if (h_per_rec)
      HIPCHK(hipMemcpyAsync(h_per_rec + (size_t)r * BT * d, H, hbytes, hipMemcpyDeviceToDevice, s));
  }
  if (middle) {
    const int last = 1 + R * n_s;
    const KeySet keys_last{kv_k(h, last), kv_vt(h, last), act_r(0), cnt_r(0)};
    st = run_layer<E>(h, h->blk[n_s + 1], H, all, kv_k(h, last), kv_vt(h, last), keys_last, B, T, s);
    if (st != MOR_OK) return st;
  }

  for (int r = 1; r <= R; ++r) {
    if (sel_pos)
      HIPCHK(hipMemcpyAsync(sel_pos + (size_t)(r - 1) * BT, act_r(r), BT * 4, hipMemcpyDeviceToDevice, s));
    if (counts)
      HIPCHK(hipMemcpyAsync(counts + (size_t)(r - 1) * B, cnt_r(r), (size_t)B * 4, hipMemcpyDeviceToDevice, s));
  }
  if (logits) {
    if (tc) {
      for (int r = 0; r < R; ++r)
        HIPCHK(hipMemcpyAsync(logits + (size_t)r * BT, h->tc_logits + (size_t)r * BT, BT * 4,
                              hipMemcpyDeviceToDevice, s));
    } else {
      for (int r = 1; r <= R; ++r)
        HIPCHK(hipMemcpyAsync(logits + (size_t)(r - 1) * BT, z_r(r), BT * 4, hipMemcpyDeviceToDevice, s));
    }
  }
  return MOR_OK;
}

// ------------------------------------------------------------------ decode iteration

// fold_in: residual partial sums of the previous layer still to be added into X (0 if X is
// already complete); fold_in < 0: the kernel before this layer already wrote its normalised
// input Xn. The layer leaves its down projection's kSplitDown partial sums, which the next
// consumer of X adds.
template <typename E>
mor_status dec_layer(mor_handle_s* h, const BlockPacked& w, int kind, int j, int fold_in, hipStream_t s) {
  const mor_config& c = h->cfg;
  const DecArgs& a = h->dec;
  const int d = c.d_model, dff = c.d_ff, S = a.S;
  E* Xn = reinterpret_cast<E*>(h->dXn);
  if (fold_in >= 0)
    HIPCHK(launch_dec_norm<E>(a, kind == DL_FIRST, kind == DL_FIRST ? 0 : fold_in, w.g_attn, c.rms_eps, Xn, s));
  SkinnyEpi eq{};
  eq.out = h->dQkv; eq.ldo = h->nqkv;
  HIPCHK(launch_skinny<E>(SK_PARTIAL, Xn, reinterpret_cast<const E*>(w.wqkv), h->nqkv, d, S, kSplitQKV, eq, s));
  HIPCHK(launch_dec_attn<E>(a, kind, j, s));
  SkinnyEpi ex{};
  ex.out = h->dPx; ex.ldo = d;
  HIPCHK(launch_skinny<E>(SK_PARTIAL, reinterpret_cast<const E*>(h->dO), reinterpret_cast<const E*>(w.wo), d, h->nq, S, kSplitO, ex, s));
  HIPCHK(launch_dec_norm<E>(a, false, kSplitO, w.g_ffn, c.rms_eps, Xn, s));
  SkinnyEpi eg{};
  eg.h = h->dHf; eg.ldh = dff;
  HIPCHK(launch_skinny<E>(SK_SWIGLU, Xn, reinterpret_cast<const E*>(w.wgu), 2 * dff, d, S, 1, eg, s));
  HIPCHK(launch_skinny<E>(SK_PARTIAL, reinterpret_cast<const E*>(h->dHf), reinterpret_cast<const E*>(w.wd), d, dff, S, kSplitDown, ex, s));
  return MOR_OK;
}

template <typename E>
mor_status dec_iteration(mor_handle_s* h, hipStream_t s) {
  const int n_s = h->n_s;
  HIPCHK(launch_dec_schedule(h->dec, s));
  mor_status st = dec_layer<E>(h, h->blk[0], DL_FIRST, 0, 0, s);
  if (st != MOR_OK) return st;
  E* Xn = reinterpret_cast<E*>(h->dXn);
  const float eps = h->cfg.rms_eps;
  // X of new tokens += first layer's down; then the first shared layer's input norm
  HIPCHK(launch_dec_prep<E>(h->dec, kSplitDown, h->blk[1].g_attn, eps, Xn, s));
  for (int j = 1; j <= n_s; ++j) {
    st = dec_layer<E>(h, h->blk[j], DL_SHARED, j, j == 1 ? -1 : kSplitDown, s);
    if (st != MOR_OK) return st;
  }
  // F(H) = X + last shared layer's down, the gated update and exit test; then the last layer's norm
  HIPCHK(launch_dec_update<E>(h->dec, kSplitDown, h->blk[n_s + 1].g_attn, eps, Xn, s));
  st = dec_layer<E>(h, h->blk[n_s + 1], DL_LAST, 0, -1, s);
  if (st != MOR_OK) return st;
  HIPCHK(launch_dec_output(h->dec, kSplitDown, s));    // output = X + last layer's down
  return MOR_OK;
}

// Iterations per captured graph, and the switch that turns graphs off (MOR_DECODE_GRAPH=0).
constexpr int kGraphIters = 8;
bool use_graph() {
  static int on = -1;
  if (on < 0) {
    const char* e = getenv("MOR_DECODE_GRAPH");
    on = (e && e[0] == '0') ? 0 : 1;
  }
  return on == 1;
}

void drop_graph(mor_handle_s* h) {
  if (h->dec_exec) (void)hipGraphExecDestroy(h->dec_exec);
  if (h->dec_graph) (void)hipGraphDestroy(h->dec_graph);
  h->dec_exec = nullptr;
  h->dec_graph = nullptr;
}

// Records kGraphIters decode iterations (fixed grids, arguments fixed per submission) on a
// private stream; the graph is then launched on the caller's stream.
mor_status capture_graph(mor_handle_s* h) {
  if (!h->cap_stream) HIPCHK(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking));
  HIPCHK(hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeRelaxed));
  mor_status st = MOR_OK;
  for (int i = 0; i < kGraphIters && st == MOR_OK; ++i)
    st = h->cfg.dtype == MOR_BF16 ? dec_iteration<bf16>(h, h->cap_stream) : dec_iteration<float>(h, h->cap_stream);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(h->cap_stream, &g);
  if (st != MOR_OK) { if (g) (void)hipGraphDestroy(g); return st; }
  if (e != hipSuccess) return fail(MOR_E_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
  h->dec_graph = g;
  HIPCHK(hipGraphInstantiate(&h->dec_exec, g, nullptr, nullptr, 0));
  return MOR_OK;
}

template <typename T>
mor_status copy_block(mor_handle_s* h, const mor_block_weights& src, const BlockPacked& dst,
                      hipStream_t s) {
  const mor_config& c = h->cfg;
  const size_t d = c.d_model, es = sizeof(T);
  const void* ptrs[] = {src.wq, src.wk, src.wv, src.wo, src.w_gate, src.w_up, src.w_down, src.g_attn, src.g_ffn};
  for (const void* p : ptrs)
    if (!p) return fail(MOR_E_INVALID, "null weight pointer");
  char* q = reinterpret_cast<char*>(dst.wqkv);
  HIPCHK(hipMemcpyAsync(q, src.wq, h->nq * d * es, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(q + h->nq * d * es, src.wk, h->nkv * d * es, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(q + (h->nq + h->nkv) * d * es, src.wv, h->nkv * d * es, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(dst.wo, src.wo, d * h->nq * es, hipMemcpyDeviceToDevice, s));
  HIPCHK(launch_pack_gate_up<T>(reinterpret_cast<const T*>(src.w_gate), reinterpret_cast<const T*>(src.w_up),
                                reinterpret_cast<T*>(dst.wgu), c.d_ff, c.d_model, s));
  HIPCHK(hipMemcpyAsync(dst.wd, src.w_down, d * c.d_ff * es, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(dst.g_attn, src.g_attn, d * 4, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(dst.g_ffn, src.g_ffn, d * 4, hipMemcpyDeviceToDevice, s));
  return MOR_OK;
}

}  // namespace

namespace {

// Binds the static scratch of mor_route_noalloc on the current device: its device address,
// looked up once per device with that device current.
mor_status scratch_on(int* dev_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOR_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOR_E_STATE, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOR_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<int*>(p);
  }
  *dev_out = dev;
  return MOR_OK;
}

}  // namespace

extern "C" {

int32_t mor_abi_version(void) { return MOR_ABI_VERSION; }

const char* mor_last_error(void) { return g_err.c_str(); }

size_t mor_workspace_bytes(const mor_config* cfg) {
  if (validate(cfg) != MOR_OK) return 0;
  return plan(*cfg, nullptr, nullptr);
}

mor_status mor_init(const mor_config* cfg, const mor_weights* w, void* workspace,
                    size_t workspace_bytes, void* stream, mor_handle** out) {
  mor_status st = validate(cfg);
  if (st != MOR_OK) return st;
  if (!w || !workspace || !out) return fail(MOR_E_INVALID, "null weights, workspace or out");
  if (!w->router_w) return fail(MOR_E_INVALID, "null router_w");
  const int n_s = shared_per_rec(*cfg);
  const bool middle = middle_sharing(*cfg);
  if (!w->shared) return fail(MOR_E_INVALID, "null shared weights");
  const size_t need = plan(*cfg, nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(MOR_E_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " + std::to_string(need));
  int dev = 0;
  st = scratch_on(&dev);
  if (st != MOR_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto* h = new mor_handle_s();
  h->cfg = *cfg;
  h->device = dev;
  char* base = reinterpret_cast<char*>(((uintptr_t)workspace + kAlign - 1) / kAlign * kAlign);
  plan(*cfg, h, base);
  auto cleanup = [&](mor_status e) { delete h; return e; };
  for (int i = 0; i < n_s + 2; ++i) {
    if (!middle && (i == 0 || i == n_s + 1)) continue;    // no unique layers to pack
    const mor_block_weights& src = i == 0 ? w->first : i == n_s + 1 ? w->last : w->shared[i - 1];
    st = cfg->dtype == MOR_BF16 ? copy_block<bf16>(h, src, h->blk[i], s) : copy_block<float>(h, src, h->blk[i], s);
    if (st != MOR_OK) return cleanup(st);
  }
  const size_t d = cfg->d_model, R = cfg->n_rec;
  hipError_t e = hipMemcpyAsync(h->router_w, w->router_w, R * d * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) {
    h->has_bias = w->router_b != nullptr;
    e = h->has_bias ? hipMemcpyAsync(h->router_b, w->router_b, R * 4, hipMemcpyDeviceToDevice, s)
                    : hipMemsetAsync(h->router_b, 0, R * 4, s);
  }
  // RoPE table: angle pos * theta^(-2i/hd), evaluated in double, stored fp32.
  const int half = cfg->head_dim / 2;
  std::vector<float> cs((size_t)cfg->max_seq * half), sn((size_t)cfg->max_seq * half);
  for (int p = 0; p < cfg->max_seq; ++p)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)cfg->rope_theta, -(2.0 * i) / cfg->head_dim);
      const double a = p * inv;
      cs[(size_t)p * half + i] = (float)std::cos(a);
      sn[(size_t)p * half + i] = (float)std::sin(a);
    }
  if (e == hipSuccess) e = hipMemcpyAsync(h->rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(h->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemsetAsync(h->err, 0, 64, s);
  // Cache slots past a sequence's active count are read (and masked) by the attention tiles;
  // zeroing the cache once keeps them finite.
  if (e == hipSuccess) e = hipMemsetAsync(h->kv, 0, h->kv_half_bytes * 2 * h->nstreams, s);
  if (e == hipSuccess && h->decode) {
    const int d = cfg->d_model;
    e = hipMemsetAsync(h->dXn, 0, 64 * (size_t)d * h->es, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->dQkv, 0, (size_t)kSplitQKV * 64 * h->nqkv * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->dPx, 0, (size_t)kSplitPx * 64 * d * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->dO, 0, 64 * (size_t)h->nq * h->es, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->dHf, 0, 64 * (size_t)cfg->d_ff * h->es, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->dec.glob, 0, G_COUNT * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->dec.sl_req, 0xFF, cfg->max_slots * 4, s);
    // every page slot holds a finite value before its first write (decode attention multiplies
    // the values of a tile's unused key slots by zero probabilities), and every page-table
    // entry a valid page
    if (e == hipSuccess) e = hipMemsetAsync(h->dec.pool, 0, (size_t)h->kv_pages * h->page_bytes, s);
    if (e == hipSuccess)
      e = hipMemsetAsync(h->dec.ptab, 0, (size_t)cfg->max_slots * h->LS * h->pps * sizeof(int), s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete h;
    return fail(MOR_E_HIP, std::string("mor_init: ") + hipGetErrorString(e));
  }
  *out = h;
  return MOR_OK;
}

mor_status mor_prefill(mor_handle* h, const float* h_in, int32_t B, int32_t T, float* h_out,
                       int32_t* sel_pos, int32_t* counts, float* logits, float* h_per_rec,
                       void* stream) {
  if (!h || !h_in || !h_out) return fail(MOR_E_INVALID, "null handle or hidden-state pointer");
  if (B < 1 || B > h->cfg.max_batch || T < 1 || T > h->cfg.max_seq)
    return fail(MOR_E_SHAPE, "B or T outside 1..max_batch / 1..max_seq");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  h->last_B = 0;
  const mor_status st = h->cfg.dtype == MOR_BF16
                            ? prefill_impl<bf16>(h, h_in, B, T, h_out, sel_pos, counts, logits, h_per_rec, s)
                            : prefill_impl<float>(h, h_in, B, T, h_out, sel_pos, counts, logits, h_per_rec, s);
  if (st == MOR_OK) { h->last_B = B; h->last_T = T; }
  return st;
}

mor_status mor_route(mor_handle* h, const float* H, const int32_t* active_in,
                     const int32_t* counts_in, int32_t r, int32_t B, int32_t T,
                     int32_t* active_out, int32_t* counts_out, float* z_out, void* stream) {
  if (!h || !H || !active_in || !counts_in || !active_out || !counts_out || !z_out)
    return fail(MOR_E_INVALID, "null pointer");
  const mor_config& c = h->cfg;
  if (c.routing == MOR_ROUTE_TOKEN_CHOICE) return fail(MOR_E_STATE, "mor_route: token choice not supported");
  if (r < 1 || r > c.n_rec) return fail(MOR_E_INVALID, "r outside 1..n_rec");
  if (B < 1 || B > c.max_batch || T < 1 || T > c.max_seq) return fail(MOR_E_SHAPE, "B or T out of range");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t MT = h->MT, BT = (size_t)B * T;
  int* meta_s = h->meta + (size_t)(c.n_rec + 1) * (c.max_batch + 1);
  HIPCHK(launch_fill_f32(z_out, BT, NAN, s));
  HIPCHK(launch_offsets(counts_in, B, meta_s, s));
  HIPCHK(launch_gather(H, c.d_model, active_in, meta_s, B, T, (int)BT, GATE_ASSIGN, nullptr, nullptr,
                       nullptr, r, h->X, h->rows, h->rows + MT, h->rows + 2 * MT, h->rows + 3 * MT,
                       h->gate, s));
  HIPCHK(launch_router(H, c.d_model, h->rows + MT, meta_s, (int)BT, h->router_w + (size_t)(r - 1) * c.d_model,
                       h->has_bias ? h->router_b + (r - 1) : nullptr, z_out, s));
  const int k = ceil_div((long)c.cap_num[r - 1] * T, c.cap_den);
  const int mode = c.routing == MOR_ROUTE_EC_TOPK ? SEL_EC : SEL_THRESHOLD;
  HIPCHK(launch_select(mode, B, T, z_out, nullptr, active_in, counts_in, k, r, active_out, counts_out, h->err, s));
  return MOR_OK;
}

mor_status mor_route_noalloc(mor_handle* h, const float* H, const int32_t* active_in,
                             const int32_t* counts_in, int32_t r, int32_t B, int32_t T,
                             int32_t* active_out, int32_t* counts_out, float* z_out, void* stream) {
  if (!h || !H || !active_in || !counts_in || !active_out || !counts_out || !z_out)
    return fail(MOR_E_INVALID, "null pointer");
  const mor_config& c = h->cfg;
  if (c.routing == MOR_ROUTE_TOKEN_CHOICE) return fail(MOR_E_STATE, "mor_route_noalloc: token choice not supported");
  if (r < 1 || r > c.n_rec) return fail(MOR_E_INVALID, "r outside 1..n_rec");
  if (B < 1 || B > c.max_batch || T < 1 || T > c.max_seq) return fail(MOR_E_SHAPE, "B or T out of range");
  if (B > MOR_NOALLOC_MAX_BATCH || (long long)B * T > MOR_NOALLOC_MAX_TOKENS)
    return fail(MOR_E_SHAPE, "mor_route_noalloc: B > " + std::to_string(MOR_NOALLOC_MAX_BATCH) +
                                 " or B*T > " + std::to_string(MOR_NOALLOC_MAX_TOKENS) +
                                 " (the static scratch holds no more); use mor_route");
  int* sp = g_scratch_ptr[h->device];
  if (!sp) return fail(MOR_E_STATE, "static scratch not bound on the handle's device");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int BT = B * T;
  int* meta = sp;                                  // [B + 1]: rows, then first row of each sequence
  int* rowsrc = sp + MOR_NOALLOC_MAX_BATCH + 1;    // [B * T]: source row of each active row
  HIPCHK(launch_fill_f32(z_out, (size_t)BT, NAN, s));
  HIPCHK(launch_offsets(counts_in, B, meta, s));
  HIPCHK(launch_rowsrc(active_in, meta, B, T, BT, rowsrc, s));
  HIPCHK(launch_router(H, c.d_model, rowsrc, meta, BT, h->router_w + (size_t)(r - 1) * c.d_model,
                       h->has_bias ? h->router_b + (r - 1) : nullptr, z_out, s));
  const int k = ceil_div((long)c.cap_num[r - 1] * T, c.cap_den);
  const int mode = c.routing == MOR_ROUTE_EC_TOPK ? SEL_EC : SEL_THRESHOLD;
  HIPCHK(launch_select(mode, B, T, z_out, nullptr, active_in, counts_in, k, r, active_out, counts_out, h->err, s));
  return MOR_OK;
}

mor_status mor_kv_view(mor_handle* h, int32_t stream, const void** k, const void** v_t,
                       int32_t* kpad) {
  if (!h || !k || !v_t || !kpad) return fail(MOR_E_INVALID, "null pointer");
  if (stream < 0 || stream >= h->nstreams) return fail(MOR_E_INVALID, "stream index out of range");
  *k = kv_k(h, stream);
  *v_t = kv_vt(h, stream);
  *kpad = h->kpad;
  return MOR_OK;
}

mor_status mor_get_error_flags(mor_handle* h, void* stream, uint32_t* flags) {
  if (!h || !flags) return fail(MOR_E_INVALID, "null pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  HIPCHK(hipMemcpyAsync(flags, h->err, 4, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  HIPCHK(hipMemsetAsync(h->err, 0, 4, s));
  HIPCHK(hipStreamSynchronize(s));
  return MOR_OK;
}

}  // extern "C"

namespace {

// Shared part of mor_decode_submit / mor_decode_continue: validates, uploads the request
// table, resets the engine; with prefix_T > 0 the requests continue the last prefill's sequences.
mor_status decode_begin(mor_handle* h, int32_t n_req, const int32_t* lengths, const float* inputs,
                        float* outputs, int8_t* exit_depth, float* h_dump, float* z_dump,
                        int prefix_T, void* stream) {
  if (!h) return fail(MOR_E_INVALID, "null handle");
  if (!h->decode) return fail(MOR_E_STATE, "handle was planned without decode state (max_slots = 0)");
  if (n_req < 1 || !lengths || !inputs || !outputs || !exit_depth)
    return fail(MOR_E_INVALID, "n_req < 1 or null pointer");
  const mor_config& c = h->cfg;
  if (n_req > c.max_requests) return fail(MOR_E_SHAPE, "n_req > max_requests");
  std::vector<int32_t> off(n_req);
  long long total = 0;
  for (int i = 0; i < n_req; ++i) {
    if (lengths[i] < 1 || prefix_T + lengths[i] > c.max_seq)
      return fail(MOR_E_SHAPE, "request length outside 1..max_seq (prefix included)");
    off[i] = (int32_t)total;
    total += lengths[i];
  }
  if (total > INT32_MAX / 2) return fail(MOR_E_SHAPE, "too many tokens in one submission");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  DecArgs& a = h->dec;
  a.inputs = inputs; a.outputs = outputs;
  a.exit_depth = reinterpret_cast<signed char*>(exit_depth);
  a.h_dump = h_dump; a.z_dump = z_dump;
  HIPCHK(hipMemcpyAsync(h->dreq_len, lengths, (size_t)n_req * 4, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(h->dreq_off, off.data(), (size_t)n_req * 4, hipMemcpyHostToDevice, s));
  if (z_dump) HIPCHK(launch_fill_f32(z_dump, (size_t)total * c.n_rec, NAN, s));
  HIPCHK(launch_dec_reset(a, n_req, s));
  if (prefix_T > 0) {
    PrefixSrc p{h->kv, h->kv_half_bytes, h->kpad, h->cnt + c.max_batch, c.max_batch, n_req, prefix_T};
    HIPCHK(launch_dec_prefix(a, p, s));
  }
  HIPCHK(hipStreamSynchronize(s));   // the host copies above read pageable memory
  drop_graph(h);                     // its kernel arguments name the previous submission's buffers
  h->submitted = true;
  return MOR_OK;
}

}  // namespace

extern "C" {

mor_status mor_decode_submit(mor_handle* h, int32_t n_req, const int32_t* lengths,
                             const float* inputs, float* outputs, int8_t* exit_depth,
                             float* h_dump, float* z_dump, void* stream) {
  return decode_begin(h, n_req, lengths, inputs, outputs, exit_depth, h_dump, z_dump, 0, stream);
}

mor_status mor_decode_continue(mor_handle* h, int32_t n_req, const int32_t* lengths,
                               const float* inputs, float* outputs, int8_t* exit_depth,
                               float* h_dump, float* z_dump, void* stream) {
  if (!h) return fail(MOR_E_INVALID, "null handle");
  if (h->cfg.routing != MOR_ROUTE_THRESHOLD || !h->decode)
    return fail(MOR_E_STATE, "decode continuation needs a threshold-routed handle with decode state");
  if (h->last_B == 0) return fail(MOR_E_STATE, "no prefill to continue on this handle");
  if (n_req != h->last_B) return fail(MOR_E_SHAPE, "n_req must equal the batch of the last prefill");
  if (n_req > h->cfg.max_slots) return fail(MOR_E_SHAPE, "n_req > max_slots");
  return decode_begin(h, n_req, lengths, inputs, outputs, exit_depth, h_dump, z_dump, h->last_T, stream);
}

mor_status mor_decode_step(mor_handle* h, int32_t n_iters, void* stream, int32_t* progress) {
  if (!h) return fail(MOR_E_INVALID, "null handle");
  if (!h->decode || !h->submitted) return fail(MOR_E_STATE, "no decode submission on this handle");
  if (n_iters < 0) return fail(MOR_E_INVALID, "n_iters < 0");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int done = 0;
  if (n_iters >= kGraphIters && use_graph()) {
    if (!h->dec_exec) {
      mor_status st = capture_graph(h);
      if (st != MOR_OK) return st;
    }
    for (; done + kGraphIters <= n_iters; done += kGraphIters) HIPCHK(hipGraphLaunch(h->dec_exec, s));
  }
  for (; done < n_iters; ++done) {
    const mor_status st = h->cfg.dtype == MOR_BF16 ? dec_iteration<bf16>(h, s) : dec_iteration<float>(h, s);
    if (st != MOR_OK) return st;
  }
  if (progress) {
    int32_t g[G_COUNT];
    uint32_t flags = 0;
    HIPCHK(hipMemcpyAsync(g, h->dec.glob, sizeof(g), hipMemcpyDeviceToHost, s));
    HIPCHK(hipMemcpyAsync(&flags, h->err, 4, hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    progress[0] = g[G_TOKENS];
    progress[1] = g[G_REQS];
    progress[2] = g[G_ITER];
    if (flags & ERR_KV_FULL) return fail(MOR_E_KV_FULL, "decode KV page pool exhausted");
  }
  return MOR_OK;
}

mor_status mor_decode_stats(mor_handle* h, void* stream, int64_t* out) {
  if (!h || !out) return fail(MOR_E_INVALID, "null pointer");
  if (!h->decode) return fail(MOR_E_STATE, "handle was planned without decode state (max_slots = 0)");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t g[G_COUNT];
  unsigned long long st[ST_COUNT];
  HIPCHK(hipMemcpyAsync(g, h->dec.glob, sizeof(g), hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(st, h->dec.stats, sizeof(st), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  out[0] = g[G_TOKENS]; out[1] = g[G_REQS]; out[2] = g[G_NEXT]; out[3] = g[G_ITER];
  for (int i = 0; i < ST_COUNT; ++i) out[4 + i] = (int64_t)st[i];
  out[8] = g[G_PEAK];
  out[9] = (int64_t)h->page_bytes;
  return MOR_OK;
}

mor_status mor_timing_enable(mor_handle* h, int32_t kind, int32_t max_launches) {
  if (!h) return fail(MOR_E_INVALID, "null handle");
  if (kind < 0 || kind > KIND_LAST || max_launches < 0) return fail(MOR_E_INVALID, "kind or max_launches");
  for (hipEvent_t e : h->ev) (void)hipEventDestroy(e);
  h->ev.clear();
  h->ev_used = 0;
  h->timing_kind = kind;
  if (h->clk) {
    const unsigned long long zero[2] = {0, 0};
    HIPCHK(hipDeviceSynchronize());
    HIPCHK(hipMemcpy(h->clk, zero, sizeof(zero), hipMemcpyHostToDevice));
  }
  if (kind == 0) return MOR_OK;
  h->ev.resize(2 * (size_t)max_launches, nullptr);
  for (auto& e : h->ev) HIPCHK(hipEventCreate(&e));
  return MOR_OK;
}

mor_status mor_timing_read(mor_handle* h, double* total_ms, int32_t* launches) {
  if (!h || !total_ms || !launches) return fail(MOR_E_INVALID, "null pointer");
  double acc = 0.0;
  if (h->ev_used) HIPCHK(hipEventSynchronize(h->ev[h->ev_used - 1]));
  for (size_t i = 0; i + 1 < h->ev_used; i += 2) {
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, h->ev[i], h->ev[i + 1]));
    acc += ms;
  }
  *total_ms = acc;
  *launches = (int32_t)(h->ev_used / 2);
  h->ev_used = 0;
  return MOR_OK;
}

mor_status mor_timing_clock(mor_handle* h, double* ghz) {
  if (!h || !ghz) return fail(MOR_E_INVALID, "null pointer");
  *ghz = 0.0;
  if (!h->clk) return MOR_OK;
  unsigned long long v[2] = {0, 0};
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemcpy(v, h->clk, sizeof(v), hipMemcpyDeviceToHost));
  int khz = 0;
  HIPCHK(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, h->device));
  if (v[1] > 0 && khz > 0) *ghz = (double)v[0] / (double)v[1] * (double)khz * 1e-6;
  return MOR_OK;
}

void mor_destroy(mor_handle* h) {
  if (!h) return;
  drop_graph(h);
  if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
  for (hipEvent_t e : h->ev) (void)hipEventDestroy(e);
  delete h;
}

}  // extern "C"
