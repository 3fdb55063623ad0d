// Dense projections of the Llama block on MFMA (gfx950): C^T = W . A^T with fp32 accumulation.
//
// A holds the active tokens' rows [M][K] (compacted per recursion), W the weights [N][K]
// ([out][in]); both are K-contiguous, so both MFMA operands load as 16-byte row pieces.
// The product is formed transposed (weights on the MFMA A side): each lane then owns four
// consecutive output columns of one token row, which gives vector stores and lets the
// epilogues see the pairs they need in registers:
//   QKV   RoPE (rotate-half pairs i, i+hd/2 of a head sit in the same lane), Q out,
//         K into the per-sequence cache, V transposed into the cache.
//   RESID fp32 residual add X += acc (the O and down projections).
//   SWIGLU gate and up rows are packed in alternating 16-row groups, so silu(gate)*up of one
//         column is formed in one lane and only the product is written.
// Tile: BN weight rows x BM tokens x (128 bytes of K) per stage, 4 waves in 2x2, LDS double
// buffered, one barrier per K step.
#include "mor_internal.h"

namespace mor {

template <typename T, int BN, int BM, int EPI>
__global__ __launch_bounds__(256) void k_gemm(const T* __restrict__ A, const T* __restrict__ W,
                                              int N, int K, const int* __restrict__ meta,
                                              GemmEpi ep) {
  constexpr int BK = 128 / (int)sizeof(T);
  constexpr int LDR = BK + 16 / (int)sizeof(T);       // LDS row, padded by 16 bytes
  constexpr int WN = BN / 2, WM = BM / 2;
  constexpr int FN = WN / 16, FM = WM / 16;
  constexpr int CH = 16 / (int)sizeof(T);             // elements per 16-byte chunk
  constexpr int PW = BN / 32, PA = BM / 32;           // 16-byte loads per thread per stage
  typedef Mma<T> MM;
  __shared__ __attribute__((aligned(16))) T sW[2][BN * LDR];
  __shared__ __attribute__((aligned(16))) T sA[2][BM * LDR];

  const int M = meta[0];
  const int m0 = blockIdx.y * BM;
  if (m0 >= M) return;
  const int n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int lr = tid >> 3, lc = (tid & 7) * CH;

  uint4 rW[PW], rA[PA];
  const T* wrow[PW];
  const T* arow[PA];
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    int n = min(n0 + p * 32 + lr, N - 1);
    wrow[p] = W + (size_t)n * K + lc;
  }
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    int m = min(m0 + p * 32 + lr, M - 1);
    arow[p] = A + (size_t)m * K + lc;
  }
  auto gload = [&](int kt) {
#pragma unroll
    for (int p = 0; p < PW; ++p) rW[p] = *reinterpret_cast<const uint4*>(wrow[p] + kt * BK);
#pragma unroll
    for (int p = 0; p < PA; ++p) rA[p] = *reinterpret_cast<const uint4*>(arow[p] + kt * BK);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PW; ++p)
      *reinterpret_cast<uint4*>(&sW[buf][(p * 32 + lr) * LDR + lc]) = rW[p];
#pragma unroll
    for (int p = 0; p < PA; ++p)
      *reinterpret_cast<uint4*>(&sA[buf][(p * 32 + lr) * LDR + lc]) = rA[p];
  };

  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * MM::KW;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / MM::KSTEP; ++ks) {
      typename MM::frag a[FN], b[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        a[i] = MM::load(&sW[cur][(wn * WN + i * 16 + fr) * LDR + ks * MM::KSTEP + fk]);
#pragma unroll
      for (int j = 0; j < FM; ++j)
        b[j] = MM::load(&sA[cur][(wm * WM + j * 16 + fr) * LDR + ks * MM::KSTEP + fk]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = MM::mma(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogues
  const int g4 = (lane >> 4) * 4;           // first of this lane's four rows of a 16-row frag
  const int nw = n0 + wn * WN;              // first weight row of this wave
  const int mw = m0 + wm * WM + fr;         // this lane's token row for frag j: mw + 16 j

  if constexpr (EPI == EPI_RESID) {
    const float* xs = ep.xin ? ep.xin : ep.x;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = mw + 16 * j;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = nw + 16 * i + g4;
        if (n >= N) continue;
        float4* px = reinterpret_cast<float4*>(ep.x + (size_t)m * ep.ldx + n);
        float4 v = *reinterpret_cast<const float4*>(xs + (size_t)m * ep.ldx + n);
        v.x += acc[i][j][0]; v.y += acc[i][j][1]; v.z += acc[i][j][2]; v.w += acc[i][j][3];
        *px = v;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = mw + 16 * j;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < FN; i += 2) {
        const int np = nw + 16 * i;         // packed row of the gate group (multiple of 32)
        if (np >= N) continue;
        const int col = (np >> 1) + g4;     // original FFN column
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float gt = acc[i][j][e], up = acc[i + 1][j][e];
          o[e] = gt / (1.f + __expf(-gt)) * up;
        }
        Vec4<T>::store(reinterpret_cast<T*>(ep.h) + (size_t)m * ep.ldh + col, o[0], o[1], o[2], o[3]);
      }
    }
  } else {  // EPI_QKV
    const int hd = ep.hd, half = hd >> 1;
    // Rotate-half partner of every accumulator, taken before any divergence.
    float pv[FN][FM][4];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (half >= 16) {
            const int c0 = (nw + 16 * i) % hd;          // column of the frag inside its head
            const int ip = (c0 < half) ? i + half / 16 : i - half / 16;
            pv[i][j][e] = (ip >= 0 && ip < FN) ? acc[ip][j][e] : 0.f;
          } else {
            pv[i][j][e] = __shfl_xor(acc[i][j][e], 32);  // hd = 16: partner is 2 lane groups away
          }
        }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = mw + 16 * j;
      if (m >= M) continue;
      const int pos = ep.rowpos[m];
      const int bseq = ep.rowseq[m], bidx = ep.rowidx[m];
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int nf = nw + 16 * i;
        if (nf >= N) continue;
        if (nf < ep.nq + ep.nkv) {          // Q or K: rotary embedding
          const int rbase = nf < ep.nq ? 0 : ep.nq;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = (nf - rbase) % hd + g4 + e;
            const int f = c % half;
            const float cs = ep.rope_cos[pos * half + f], sn = ep.rope_sin[pos * half + f];
            const float x = acc[i][j][e], p = pv[i][j][e];
            o[e] = c < half ? x * cs - p * sn : x * cs + p * sn;
          }
          if (nf < ep.nq) {
            Vec4<T>::store(reinterpret_cast<T*>(ep.q) + (size_t)m * ep.ldq + nf + g4, o[0], o[1], o[2], o[3]);
          } else {
            T* kp = reinterpret_cast<T*>(ep.k) + ((size_t)bseq * ep.kpad + bidx) * ep.nkv + (nf - ep.nq) + g4;
            Vec4<T>::store(kp, o[0], o[1], o[2], o[3]);
          }
        } else {                            // V: transposed into the cache
          const int vn = nf - ep.nq - ep.nkv + g4;
          const int kvh = vn / hd, dc = vn % hd;
          T* vp = reinterpret_cast<T*>(ep.vt) + (((size_t)bseq * ep.hkv + kvh) * hd + dc) * ep.kpad + bidx;
#pragma unroll
          for (int e = 0; e < 4; ++e) vp[(size_t)e * ep.kpad] = from_f32<T>(acc[i][j][e]);
        }
      }
    }
  }
}

template <typename T, int BN, int BM>
static hipError_t launch_tile(int epi, const T* A, const T* W, int N, int K, int m_upper,
                              const int* meta, const GemmEpi& ep, hipStream_t s) {
  dim3 grid((N + BN - 1) / BN, (m_upper + BM - 1) / BM);
  if (grid.y == 0) return hipSuccess;
  switch (epi) {
    case EPI_QKV: hipLaunchKernelGGL((k_gemm<T, BN, BM, EPI_QKV>), grid, dim3(256), 0, s, A, W, N, K, meta, ep); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemm<T, BN, BM, EPI_RESID>), grid, dim3(256), 0, s, A, W, N, K, meta, ep); break;
    default: hipLaunchKernelGGL((k_gemm<T, BN, BM, EPI_SWIGLU>), grid, dim3(256), 0, s, A, W, N, K, meta, ep); break;
  }
  return hipGetLastError();
}

// fp32 configurations use this kernel; bf16 uses the tuned kernel in k_gemm_bf16.hip.
template <>
hipError_t launch_gemm<float>(int epi, const float* A, const float* W, int N, int K, int m_upper,
                              const int* meta, const GemmEpi& ep, hipStream_t s) {
  return launch_tile<float, 128, 128>(epi, A, W, N, K, m_upper, meta, ep, s);
}

}  // namespace mor
