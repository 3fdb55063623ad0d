// Routing, compaction, gated scatter and RMSNorm kernels (gfx950, wave64).
//
// Router logits (reading notes 2.1: g = sigmoid(theta_r^T H); 2.2: softmax(Theta^T H^1)) are
// fp32 dot products in one fixed order (fold_fixed in mor_device.h), so the same H gives the
// same bits on any run and in the reference. Expert-choice keeps, per sequence, the
// ceil(cap_r * T) tokens of the previous active set with the largest logits (ties: lower
// position), found by an MSB-first 8-bit radix select over order-preserving keys; the
// threshold and token-choice modes keep tokens by a per-token test. The kept tokens are
// written in position order by wave ballots and a workgroup prefix sum.
#include <climits>
#include "mor_internal.h"

namespace mor {

// ------------------------------------------------------------------ identity row sets
__global__ void k_init_sets(int B, int T, int* act0, int* cnt0, int* meta0, int* rowpos,
                            int* rowsrc, int* rowseq, int* rowidx) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B * T) {
    const int b = i / T, t = i - b * T;
    act0[i] = t;
    rowpos[i] = t;
    rowsrc[i] = i;
    rowseq[i] = b;
    rowidx[i] = t;
  }
  if (i < B) cnt0[i] = T;
  if (i <= B) meta0[i] = (i == 0) ? B * T : (i - 1) * T;
}

hipError_t launch_init_sets(int B, int T, int* act0, int* cnt0, int* meta0, int* rowpos,
                            int* rowsrc, int* rowseq, int* rowidx, hipStream_t s) {
  const int n = B * T > B + 1 ? B * T : B + 1;
  hipLaunchKernelGGL(k_init_sets, dim3((n + 255) / 256), dim3(256), 0, s, B, T, act0, cnt0,
                     meta0, rowpos, rowsrc, rowseq, rowidx);
  return hipGetLastError();
}

// ------------------------------------------------------------------ router logits
// One wave per active row: z[src] = w . H[src] (+ bias), fixed order.
__global__ __launch_bounds__(256) void k_router(const float* __restrict__ H, int d,
                                                const int* __restrict__ rowsrc,
                                                const int* __restrict__ meta,
                                                const float* __restrict__ w,
                                                const float* __restrict__ bias,
                                                float* __restrict__ z) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (row >= meta[0]) return;
  const int src = rowsrc[row];
  const float* h = H + (size_t)src * d;
  float p = 0.f;
  for (int i = lane; i < d; i += WAVE) p = add_rn(p, mul_rn(h[i], w[i]));
  p = fold_fixed(p);
  if (bias) p = add_rn(p, bias[0]);
  if (lane == 0) z[src] = (p == 0.f) ? 0.f : p;
}

hipError_t launch_router(const float* H, int d, const int* rowsrc, const int* meta, int m_upper,
                         const float* w, const float* bias, float* z, hipStream_t s) {
  if (m_upper <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_router, dim3((m_upper + 3) / 4), dim3(256), 0, s, H, d, rowsrc, meta, w,
                     bias, z);
  return hipGetLastError();
}

// Token choice: logits[j][t] = Theta_j . H[t], depth = 1 + argmax_j (first maximum),
// prob = softmax weight of the chosen depth.
__global__ __launch_bounds__(256) void k_router_tc(const float* __restrict__ H, int d, int BT,
                                                   const float* __restrict__ W, int R,
                                                   float* __restrict__ logits,
                                                   int* __restrict__ depth,
                                                   float* __restrict__ prob) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (row >= BT) return;
  const float* h = H + (size_t)row * d;
  float zs[MOR_MAX_REC_DEV];
  float best = 0.f;
  int arg = 0;
  for (int j = 0; j < R; ++j) {
    const float* w = W + (size_t)j * d;
    float p = 0.f;
    for (int i = lane; i < d; i += WAVE) p = add_rn(p, mul_rn(h[i], w[i]));
    p = fold_fixed(p);
    p = (p == 0.f) ? 0.f : p;
    zs[j] = p;
    if (j == 0 || p > best) { best = p; arg = j; }
  }
  if (lane == 0) {
    float den = 0.f;
    for (int j = 0; j < R; ++j) den += __expf(zs[j] - best);
    for (int j = 0; j < R; ++j) logits[(size_t)j * BT + row] = zs[j];
    depth[row] = arg + 1;
    prob[row] = 1.f / den;                 // exp(z_arg - max) = 1
  }
}

hipError_t launch_router_tc(const float* H, int d, int BT, const float* W, int R, float* logits,
                            int* depth, float* prob, hipStream_t s) {
  if (R > MOR_MAX_REC_DEV) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_router_tc, dim3((BT + 3) / 4), dim3(256), 0, s, H, d, BT, W, R, logits,
                     depth, prob);
  return hipGetLastError();
}

// ------------------------------------------------------------------ selection + compaction
// Order-preserving key: smaller key = better token (larger z). -0 is +0; NaN ranks last.
__device__ __forceinline__ unsigned rank_key(float z, unsigned* err) {
  if (z != z) {
    atomicOr(err, 1u);
    return 0xFFFFFFFFu;
  }
  if (z == 0.f) z = 0.f;
  unsigned u = __float_as_uint(z);
  unsigned asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // ascending in z
  return ~asc;                                                 // ascending in -z
}

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / WAVE;

// Exclusive prefix over the workgroup of a per-thread 0/1 flag, in thread order.
// Returns this thread's rank; *total receives the number of set flags.
__device__ __forceinline__ int block_rank(bool flag, int* swave, int* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const unsigned long long below = (lane == 0) ? 0ull : (bal & ((~0ull) >> (64 - lane)));
  const int in_wave = __popcll(below);
  __syncthreads();
  if (lane == 0) swave[wave] = __popcll(bal);
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < SEL_WAVES; ++w) {
    const int c = swave[w];
    if (w < wave) base += c;
    tot += c;
  }
  *total = tot;
  return base + in_wave;
}

// One workgroup per sequence. act_prev/cnt_prev: the set active at r-1 (positions ascending).
__global__ __launch_bounds__(SEL_THREADS) void k_select(int mode, int T, const float* __restrict__ z,
                                                        const int* __restrict__ depth,
                                                        const int* __restrict__ act_prev,
                                                        const int* __restrict__ cnt_prev, int k,
                                                        int r, int* __restrict__ act_out,
                                                        int* __restrict__ cnt_out,
                                                        unsigned* __restrict__ err) {
  extern __shared__ unsigned skey[];                  // [T] rank keys of the active tokens
  __shared__ int hist[256];
  __shared__ int swave[SEL_WAVES];
  __shared__ unsigned s_prefix;
  __shared__ int s_remaining;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n = cnt_prev[b];
  const int* ap = act_prev + (size_t)b * T;
  int* ao = act_out + (size_t)b * T;
  const float* zb = z + (size_t)b * T;

  unsigned kstar = 0;
  int need_ties = 0;
  if (mode == SEL_EC) {
    const int kk = k < n ? k : n;
    for (int i = tid; i < n; i += SEL_THREADS) skey[i] = rank_key(zb[ap[i]], err);
    if (tid == 0) { s_prefix = 0; s_remaining = kk; }
    __syncthreads();
    if (kk > 0 && kk < n) {
      unsigned pmask = 0;
      for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
        __syncthreads();
        const unsigned prefix = s_prefix;
        const int rem = s_remaining;
        for (int i = tid; i < n; i += SEL_THREADS) {
          const unsigned key = skey[i];
          if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        // the digit is the first bin whose inclusive count reaches rem: a scan of the 256 bins
        // by waves 0-3 (shuffles within a wave, then the wave totals)
        const int lane = tid & 63, wave = tid >> 6;
        int hv = 0, incl = 0;
        if (tid < 256) {
          hv = hist[tid];
          incl = hv;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
          }
          if (lane == 63) swave[wave] = incl;
        }
        __syncthreads();
        if (tid < 256) {
          for (int w = 0; w < wave; ++w) incl += swave[w];
          const int excl = incl - hv;
          if (excl < rem && incl >= rem) {
            s_remaining = rem - excl;
            s_prefix = prefix | ((unsigned)tid << shift);
          }
        }
        pmask |= 255u << shift;
        __syncthreads();
      }
      kstar = s_prefix;            // the kk-th smallest key
      need_ties = s_remaining;     // how many tokens with key == kstar to keep (lowest positions)
    } else {
      kstar = (kk == 0) ? 0u : 0xFFFFFFFFu;
      need_ties = (kk == 0) ? 0 : n;   // keep all (every key <= 0xFFFFFFFF) or none
    }
    __syncthreads();
  }

  int out_base = 0, tie_base = 0;
  for (int c0 = 0; c0 < n; c0 += SEL_THREADS) {
    const int i = c0 + tid;
    const bool valid = i < n;
    const int pos = valid ? ap[i] : 0;
    bool keep = false;
    if (mode == SEL_EC) {
      const unsigned key = valid ? skey[i] : 0xFFFFFFFFu;
      const bool tie = valid && key == kstar;
      int ntie;
      const int trank = tie_base + block_rank(tie, swave, &ntie);
      tie_base += ntie;
      keep = valid && (key < kstar || (tie && trank < need_ties));
      if (k >= n) keep = valid;
      if (k <= 0) keep = false;
    } else if (mode == SEL_THRESHOLD) {
      keep = valid && (r == 1 || zb[pos] > 0.f);
    } else {
      keep = valid && depth[(size_t)b * T + pos] >= r;
    }
    int nkeep;
    const int rank = out_base + block_rank(keep, swave, &nkeep);
    if (keep) ao[rank] = pos;
    out_base += nkeep;
  }
  for (int i = out_base + tid; i < T; i += SEL_THREADS) ao[i] = -1;
  if (tid == 0) cnt_out[b] = out_base;
}

hipError_t launch_select(int mode, int B, int T, const float* z, const int* depth,
                         const int* act_prev, const int* cnt_prev, int k, int r, int* act_out,
                         int* cnt_out, unsigned* err, hipStream_t s) {
  const size_t lds = (mode == SEL_EC) ? (size_t)T * sizeof(unsigned) : 0;
  hipLaunchKernelGGL(k_select, dim3(B), dim3(SEL_THREADS), lds, s, mode, T, z, depth, act_prev,
                     cnt_prev, k, r, act_out, cnt_out, err);
  return hipGetLastError();
}

// meta[0] = sum cnt, meta[1 + b] = exclusive prefix of cnt.
__global__ void k_offsets(const int* cnt, int B, int* meta) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    int acc = 0;
    for (int b = 0; b < B; ++b) { meta[1 + b] = acc; acc += cnt[b]; }
    meta[0] = acc;
  }
}

hipError_t launch_offsets(const int* cnt, int B, int* meta, hipStream_t s) {
  hipLaunchKernelGGL(k_offsets, dim3(1), dim3(64), 0, s, cnt, B, meta);
  return hipGetLastError();
}

// Source row b*T + pos of every row of a compacted set (one thread per row), for callers that
// need the row map without the gathered copy of H.
__global__ __launch_bounds__(256) void k_rowsrc(const int* __restrict__ act, const int* __restrict__ meta,
                                                int B, int T, int* __restrict__ rowsrc) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= meta[0]) return;
  int lo = 0, hi = B - 1;                          // last b with meta[1+b] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (meta[1 + mid] <= i) lo = mid; else hi = mid - 1;
  }
  rowsrc[i] = lo * T + act[(size_t)lo * T + (i - meta[1 + lo])];
}

hipError_t launch_rowsrc(const int* act, const int* meta, int B, int T, int m_upper, int* rowsrc,
                         hipStream_t s) {
  if (m_upper <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rowsrc, dim3((m_upper + 255) / 256), dim3(256), 0, s, act, meta, B, T, rowsrc);
  return hipGetLastError();
}

// ------------------------------------------------------------------ gather / scatter
// One wave per compacted row i: find its sequence, copy H[src] into X[i], record the row maps
// and the gate of the recursion update (negative gate = plain assignment).
__global__ __launch_bounds__(256) void k_gather(const float* __restrict__ H, int d,
                                                const int* __restrict__ act,
                                                const int* __restrict__ meta, int B, int T,
                                                int gate_kind, const float* __restrict__ z,
                                                const int* __restrict__ depth,
                                                const float* __restrict__ prob, int r,
                                                float* __restrict__ X, int* __restrict__ rowpos,
                                                int* __restrict__ rowsrc, int* __restrict__ rowseq,
                                                int* __restrict__ rowidx, float* __restrict__ gate) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (i >= meta[0]) return;
  int lo = 0, hi = B - 1;                          // last b with meta[1+b] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (meta[1 + mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int b = lo, j = i - meta[1 + b];
  const int pos = act[(size_t)b * T + j];
  const int src = b * T + pos;
  const float4* hs = reinterpret_cast<const float4*>(H + (size_t)src * d);
  float4* xd = reinterpret_cast<float4*>(X + (size_t)i * d);
  const int n4 = d / 4;
  if (n4 <= 4 * WAVE) {                  // rows up to 1024: every load before the first store
    float4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = hs[min(lane + k * WAVE, n4 - 1)];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (lane + k * WAVE < n4) xd[lane + k * WAVE] = v[k];
  } else {
    for (int c = lane; c < n4; c += WAVE) xd[c] = hs[c];
  }
  if (lane == 0) {
    rowpos[i] = pos;
    rowsrc[i] = src;
    rowseq[i] = b;
    rowidx[i] = j;
    float gv;
    if (gate_kind == GATE_SIGMOID) gv = 1.f / (1.f + __expf(-z[src]));
    else if (gate_kind == GATE_TC) gv = (depth[src] == r) ? prob[src] : -1.f;
    else gv = -1.f;
    gate[i] = gv;
  }
}

hipError_t launch_gather(const float* H, int d, const int* act, const int* meta, int B, int T,
                         int m_upper, int gate_kind, const float* z, const int* depth,
                         const float* prob, int r, float* X, int* rowpos, int* rowsrc,
                         int* rowseq, int* rowidx, float* gate, hipStream_t s) {
  if (m_upper <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather, dim3((m_upper + 3) / 4), dim3(256), 0, s, H, d, act, meta, B, T,
                     gate_kind, z, depth, prob, r, X, rowpos, rowsrc, rowseq, rowidx, gate);
  return hipGetLastError();
}

// One wave per compacted row: H[src] <- H[src] + g (X[i] - H[src]) (g < 0: H[src] <- X[i]),
// then, if w_next is given, the next recursion's router logit of the updated row (fixed order:
// lane l sums elements l, l + 64, ... ascending). With CH > 0 (d <= 64 CH) every element of the
// lane is loaded before any is used (one memory round trip per row); CH = 0 loops.
template <int CH>
__global__ __launch_bounds__(256) void k_scatter(float* __restrict__ H, const float* __restrict__ X,
                                                 int d, const int* __restrict__ meta,
                                                 const int* __restrict__ rowsrc,
                                                 const float* __restrict__ gate,
                                                 const float* __restrict__ w_next,
                                                 const float* __restrict__ bias_next,
                                                 float* __restrict__ z_next) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (i >= meta[0]) return;
  const int src = rowsrc[i];
  const float g = gate[i];
  float* h = H + (size_t)src * d;
  const float* x = X + (size_t)i * d;
  float p = 0.f;
  if constexpr (CH > 0) {
    float hv[CH], xv[CH], wv[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int c = min(lane + k * WAVE, d - 1);    // loads clamped in range, stores guarded
      hv[k] = h[c];
      xv[k] = x[c];
      wv[k] = w_next ? w_next[c] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int c = lane + k * WAVE;
      if (c < d) {
        const float hn = (g < 0.f) ? xv[k] : hv[k] + g * (xv[k] - hv[k]);
        h[c] = hn;
        if (w_next) p = add_rn(p, mul_rn(hn, wv[k]));
      }
    }
  } else {
    for (int c = lane; c < d; c += WAVE) {
      const float hv = h[c], xv = x[c];
      const float hn = (g < 0.f) ? xv : hv + g * (xv - hv);
      h[c] = hn;
      if (w_next) p = add_rn(p, mul_rn(hn, w_next[c]));
    }
  }
  if (w_next) {
    p = fold_fixed(p);
    if (bias_next) p = add_rn(p, bias_next[0]);
    if (lane == 0) z_next[src] = (p == 0.f) ? 0.f : p;
  }
}

hipError_t launch_scatter(float* H, const float* X, int d, const int* meta, int m_upper,
                          const int* rowsrc, const float* gate, const float* w_next,
                          const float* bias_next, float* z_next, hipStream_t s) {
  if (m_upper <= 0) return hipSuccess;
  const dim3 grid((m_upper + 3) / 4), blk(256);
  if (d <= 16 * WAVE)
    hipLaunchKernelGGL(k_scatter<16>, grid, blk, 0, s, H, X, d, meta, rowsrc, gate, w_next, bias_next, z_next);
  else
    hipLaunchKernelGGL(k_scatter<0>, grid, blk, 0, s, H, X, d, meta, rowsrc, gate, w_next, bias_next, z_next);
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm
// One wave per row: Xn = X / sqrt(mean(X^2) + eps) * g, rounded to the GEMM input type.
// m_upper bounds the row count meta[0] (rows below it are allocated): with CH > 0 the row and
// the gains are loaded before the row count is known (row index clamped below m_upper), so the
// kernel waits for one memory round trip, not three.
template <typename T, int CH>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ X, int d,
                                                 const int* __restrict__ meta, int m_upper,
                                                 const float* __restrict__ g, float eps,
                                                 T* __restrict__ Xn) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const int n4 = d / 4;
  if constexpr (CH > 0) {
    // the row stays in registers (CH float4 per lane): one read of X
    const float4* x = reinterpret_cast<const float4*>(X + (size_t)min(i, m_upper - 1) * d);
    float4 v[CH], gg[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int c = min(lane + k * WAVE, n4 - 1);
      v[k] = x[c];
      gg[k] = g4[c];
    }
    if (i >= meta[0]) return;
    T* out = Xn + (size_t)i * d;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      if (lane + k * WAVE >= n4) v[k] = float4{0.f, 0.f, 0.f, 0.f};
      ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    }
    ss = wave_sum(ss);
    const float rinv = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int c = lane + k * WAVE;
      if (c < n4)
        Vec4<T>::store(out + 4 * c, v[k].x * rinv * gg[k].x, v[k].y * rinv * gg[k].y,
                       v[k].z * rinv * gg[k].z, v[k].w * rinv * gg[k].w);
    }
  } else {
    if (i >= meta[0]) return;
    const float4* x = reinterpret_cast<const float4*>(X + (size_t)i * d);
    T* out = Xn + (size_t)i * d;
    float ss = 0.f;
    for (int c = lane; c < n4; c += WAVE) {
      const float4 v = x[c];
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    const float rinv = 1.f / sqrtf(ss / (float)d + eps);
    for (int c = lane; c < n4; c += WAVE) {
      const float4 v = x[c], gg = g4[c];
      Vec4<T>::store(out + 4 * c, v.x * rinv * gg.x, v.y * rinv * gg.y, v.z * rinv * gg.z,
                     v.w * rinv * gg.w);
    }
  }
}

template <typename T>
hipError_t launch_rmsnorm(const float* X, int d, const int* meta, int m_upper, const float* g,
                          float eps, T* Xn, hipStream_t s) {
  if (m_upper <= 0) return hipSuccess;
  const dim3 grid((m_upper + 3) / 4);
  if (d <= 4 * 4 * WAVE)
    hipLaunchKernelGGL((k_rmsnorm<T, 4>), grid, dim3(256), 0, s, X, d, meta, m_upper, g, eps, Xn);
  else
    hipLaunchKernelGGL((k_rmsnorm<T, 0>), grid, dim3(256), 0, s, X, d, meta, m_upper, g, eps, Xn);
  return hipGetLastError();
}
template hipError_t launch_rmsnorm<float>(const float*, int, const int*, int, const float*, float, float*, hipStream_t);
template hipError_t launch_rmsnorm<bf16>(const float*, int, const int*, int, const float*, float, bf16*, hipStream_t);

// ------------------------------------------------------------------ small utilities
__global__ void k_fill_f32(float* p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// Packs gate and up rows in alternating groups of 16 ([gate 16q..16q+15][up 16q..16q+15] ...),
// the layout the SwiGLU epilogue reads.
template <typename T>
__global__ void k_pack_gate_up(const T* __restrict__ wg, const T* __restrict__ wu, T* __restrict__ out,
                               int d) {
  const int n = blockIdx.x;
  const int q = n >> 5, w = n & 31;
  const T* src = ((w < 16) ? wg : wu) + (size_t)(16 * q + (w & 15)) * d;
  T* dst = out + (size_t)n * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) dst[c] = src[c];
}

template <typename T>
hipError_t launch_pack_gate_up(const T* wg, const T* wu, T* out, int dff, int d, hipStream_t s) {
  hipLaunchKernelGGL((k_pack_gate_up<T>), dim3(2 * dff), dim3(256), 0, s, wg, wu, out, d);
  return hipGetLastError();
}
template hipError_t launch_pack_gate_up<float>(const float*, const float*, float*, int, int, hipStream_t);
template hipError_t launch_pack_gate_up<bf16>(const bf16*, const bf16*, bf16*, int, int, hipStream_t);

}  // namespace mor
