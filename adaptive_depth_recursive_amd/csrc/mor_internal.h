// Internal interface between the host runtime (mor_api.hip) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mor_device.h"

namespace mor {

enum { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };

// Arguments of the GEMM epilogues (unused fields are ignored by the other epilogues).
struct GemmEpi {
  // EPI_QKV
  void* q; int ldq;                 // Q out [M][nq]
  void* k; void* vt;                // K cache [B][kpad][nkv]; V^T cache [B][hkv][hd][kpad]
  int nq, nkv, hd, hkv, kpad;
  const int* rowpos;                // original position of every row (RoPE)
  const int* rowseq;                // sequence of every row
  const int* rowidx;                // index of the row inside its sequence's active list
  const float* rope_cos;            // [max_seq][hd/2]
  const float* rope_sin;
  // EPI_RESID: x[m][n] = xin[m][n] + acc (xin == nullptr: x is read and written in place)
  float* x; int ldx;
  const float* xin;
  // EPI_SWIGLU
  void* h; int ldh;
  // host side: the launch's row count is only an upper bound (the rows are counted on the
  // device), so the tile choice avoids tiles of one workgroup per CU
  int rows_bound;
  // measurement hook (bf16 kernel): when set, the first workgroup adds its shader cycles and
  // real-time counter ticks over its life to clk[0] and clk[1]
  unsigned long long* clk;
};

// Row-set descriptor ("meta"): meta[0] = total rows M, meta[1 + b] = first row of sequence b.
template <typename T>
hipError_t launch_gemm(int epi, const T* A, const T* W, int N, int K, int m_upper,
                       const int* meta, const GemmEpi& ep, hipStream_t s);

struct AttnArgs {
  const void* q; int ldq;           // [M][Hq*hd]
  const int* qmeta;                 // row-set descriptor of the queries
  const int* qcnt;                  // [B] queries per sequence
  const int* qpos;                  // [M] original positions of the queries
  const void* k; const void* vt;    // cache stream read by this layer
  const int* kpos; int ldkpos;      // [B][ldkpos] positions of the cached tokens (ascending)
  const int* kcnt;                  // [B] cached tokens per sequence
  int kpad, hkv, hq, hd;
  void* o; int ldo;                 // [M][Hq*hd]
  float scale_log2;                 // log2(e) / sqrt(hd)
};
template <typename T>
hipError_t launch_attention(const AttnArgs& a, int B, int max_rows_per_seq, hipStream_t s);
// bf16, head_dim 64 (k_attn_bf16.hip); grid = (query blocks of 64, B, Hkv).
hipError_t launch_attention_bf16(const AttnArgs& a, dim3 grid, hipStream_t s);

// Routing, compaction, scatter and normalisation kernels (k_route.hip).
hipError_t launch_init_sets(int B, int T, int* act0, int* cnt0, int* meta0, int* rowpos,
                            int* rowsrc, int* rowseq, int* rowidx, hipStream_t s);
hipError_t launch_router(const float* H, int d, const int* rowsrc, const int* meta, int m_upper,
                         const float* w, const float* bias, float* z, hipStream_t s);
hipError_t launch_router_tc(const float* H, int d, int BT, const float* W, int R, float* logits,
                            int* depth, float* prob, hipStream_t s);
enum { SEL_EC = 0, SEL_THRESHOLD = 1, SEL_TC = 2 };
hipError_t launch_select(int mode, int B, int T, const float* z, const int* depth,
                         const int* act_prev, const int* cnt_prev, int k, int r, int* act_out,
                         int* cnt_out, unsigned* err, hipStream_t s);
hipError_t launch_offsets(const int* cnt, int B, int* meta, hipStream_t s);
hipError_t launch_rowsrc(const int* act, const int* meta, int B, int T, int m_upper, int* rowsrc,
                         hipStream_t s);
enum { GATE_SIGMOID = 0, GATE_ASSIGN = 1, GATE_TC = 2 };
hipError_t launch_gather(const float* H, int d, const int* act, const int* meta, int B, int T,
                         int m_upper, int gate_kind, const float* z, const int* depth,
                         const float* prob, int r, float* X, int* rowpos, int* rowsrc,
                         int* rowseq, int* rowidx, float* gate, hipStream_t s);
hipError_t launch_scatter(float* H, const float* X, int d, const int* meta, int m_upper,
                          const int* rowsrc, const float* gate, const float* w_next,
                          const float* bias_next, float* z_next, hipStream_t s);
template <typename T>
hipError_t launch_rmsnorm(const float* X, int d, const int* meta, int m_upper, const float* g,
                          float eps, T* Xn, hipStream_t s);
hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t s);
template <typename T>
hipError_t launch_pack_gate_up(const T* wg, const T* wu, T* out, int dff, int d, hipStream_t s);

}  // namespace mor

// ------------------------------------------------------------------ depth-wise batched decode
namespace mor {

// Indices of the engine's global counters (DecArgs::glob).
enum { G_NEXT = 0, G_TOP = 1, G_TOKENS = 2, G_REQS = 3, G_HALT = 4, G_NREQ = 5, G_ITER = 6,
       G_PEAK = 7, G_COUNT = 16 };  // G_PEAK: most pages in use at once
// Error flag bits (shared with prefill's bit 0 = NaN router logit).
enum { ERR_NAN_LOGIT = 1u, ERR_KV_FULL = 2u };
// Layer kinds of one decode iteration: which slots take part and which cache stream they use.
enum { DL_FIRST = 0, DL_SHARED = 1, DL_LAST = 2 };

// Everything the decode kernels read or write. Slots are the rows of every decode GEMM (at most
// 64, padded to 64 rows); a slot holds one request, and at most one of its tokens is in flight.
// K splits of the decode QKV projection that decode attention folds (at most).
constexpr int kMaxQkvSplits = 4;

struct DecArgs {
  int S, R, n_s, P, pps, LS;           // slots, N_r, shared layers, page tokens, pages per stream, layer streams
  int d, hd, hkv, hq, nq, nkv, nqkv;
  int kv_share, unit_gate;
  long long page_elems;                // elements of one page: K then V, each [hkv][P][hd]
  int kv_pages;
  // slot table
  int* sl_req;                         // request in the slot, -1 = free
  int* sl_pos;                         // index of the token in flight within the request
  int* sl_base;                        // cached prefix of the request (its tokens sit at base + pos)
  int* sl_depth;                       // recursion the token runs this iteration (0 = token finished)
  int* sl_first;                       // token admitted this iteration (runs the first layer)
  int* sl_part;                        // slot runs the shared block this iteration
  int* sl_exit;                        // token leaves after this iteration's recursion (runs the last layer)
  int* sl_cnt;                         // [S][R] tokens of the request that completed recursion r
  int* ptab;                           // [S][LS][pps] page of (slot, layer stream, page index)
  int* free_pages;                     // [kv_pages] stack of free pages
  int* glob;                           // [G_COUNT]
  unsigned* err;
  const int* req_len;                  // [n_req]
  const int* req_off;                  // [n_req] first row of the request in inputs/outputs
  const float* inputs;                 // [tokens][d]
  float* outputs;                      // [tokens][d]
  signed char* exit_depth;             // [tokens]
  float* h_dump;                       // [tokens][R+1][d] or null
  float* z_dump;                       // [tokens][R] or null
  float* X;                            // [64][d] working rows
  float* Hs;                           // [64][d] state of each slot at the start of its recursion
  float* gate;                         // [64]
  const float* router_w;               // [R][d]
  const float* router_b;               // [R]
  const float* rope_cos;               // [max_seq][hd/2]
  const float* rope_sin;
  void* pool;                          // KV pages
  const float* qkv;                    // [kqkv][64][nqkv] fp32 partial sums of the QKV projection
  int kqkv;                            // K splits of the QKV projection
  const float* px;                     // [<=8][64][d] fp32 partial sums of the O / down projections
  void* o;                             // [64][nq] attention output
  float scale_log2;
  // algorithmic bytes of the iterations (measurement): weights of every layer that runs, K/V
  // read and appended by the participating slots, input and output rows
  unsigned long long* stats;           // [ST_COUNT]
  long long layer_weight_bytes;
  int es;                              // bytes per element of the weights and the cache
};
enum { ST_WEIGHT = 0, ST_KV_READ = 1, ST_KV_WRITE = 2, ST_ACT = 3, ST_COUNT = 4 };

hipError_t launch_dec_schedule(const DecArgs& a, hipStream_t s);
// `fold` = number of residual partial sums (DecArgs::px) to add into X before the kernel's work.
template <typename T>
hipError_t launch_dec_norm(const DecArgs& a, bool gather_inputs, int fold, const float* g,
                           float eps, T* Xn, hipStream_t s);
// prep and update also do the RMSNorm (gain, eps) of every slot row into Xn for the layer that
// follows them.
template <typename T>
hipError_t launch_dec_prep(const DecArgs& a, int fold, const float* gain, float eps, T* Xn, hipStream_t s);
template <typename T>
hipError_t launch_dec_update(const DecArgs& a, int fold, const float* gain, float eps, T* Xn, hipStream_t s);
hipError_t launch_dec_output(const DecArgs& a, int fold, hipStream_t s);
template <typename T>
hipError_t launch_dec_attn(const DecArgs& a, int kind, int j, hipStream_t s);
hipError_t launch_dec_reset(const DecArgs& a, int n_req, hipStream_t s);
// Hand-over from a prefill: slot b takes request b with the T-token prefix of prefill sequence b.
// `streams` points at the prefill cache streams (K [B][kpad][hkv][hd], V^T [B][hkv][hd][kpad]),
// `cnt` at the prefill's per-recursion counts [N_r][max_batch].
struct PrefixSrc {
  const void* kv; size_t half_bytes; int kpad; const int* cnt; int cnt_ld; int B; int T;
};
hipError_t launch_dec_prefix(const DecArgs& a, const PrefixSrc& p, hipStream_t s);

// Skinny projections of the decode batch: out^T = W . A^T for the 64 slot rows of A.
//  SK_PARTIAL: K is split over `ksplit` workgroup rows; split k writes its fp32 partial sum to
//              out + k * 64 * ldo ([64][ldo]); the consumer adds the splits in order.
//  SK_SWIGLU:  one split; SiLU(gate) * up in the element type into h [64][ldh].
enum { SK_PARTIAL = 0, SK_SWIGLU = 2 };
struct SkinnyEpi {
  float* out; int ldo;
  void* h; int ldh;
};
template <typename T>
hipError_t launch_skinny(int epi, const T* A, const T* W, int N, int K, int M, int ksplit,
                         const SkinnyEpi& ep, hipStream_t s);

}  // namespace mor
