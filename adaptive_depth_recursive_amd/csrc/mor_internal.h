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
  // EPI_RESID
  float* x; int ldx;
  // EPI_SWIGLU
  void* h; int ldh;
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
