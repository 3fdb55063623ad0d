// Causal attention over per-recursion active sets, flash-style, on MFMA (gfx950).
//
// Recursion-wise caching (MoR paper A.3; reading notes 3.1): at a recursion, a query token
// attends only to tokens active at the same recursion whose original position is not larger
// than its own. Recursive KV sharing (reading notes 3.2): it attends to the recursion-1 tokens
// instead. Both are "key s is visible to query t iff kpos[s] <= qpos[t]" over a sorted list of
// cached tokens, so one kernel serves both, driven by the position lists.
//
// Work item: (query block of 64 active tokens of one sequence, one KV head); its 4 waves hold
// 16 queries each for all Hq/Hkv query heads that share the KV head (GQA), so every K/V tile
// staged in LDS is used by all of them. Scores are formed transposed, S^T = K Q^T, so a lane
// owns one query column and 4 keys of each 16-key group; softmax statistics are reduced over
// the 4 lanes of a column. P^T then feeds the PV product directly as the MFMA B operand, with V
// stored transposed in the cache as the A operand (the same key permutation on both sides).
// Unnormalised probabilities are rounded to the element type for PV; the normaliser sums them
// in fp32.
#include <climits>
#include "mor_internal.h"

namespace mor {

template <typename T, int HD, int G>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  constexpr int BQ = 64, BKV = 64;
  constexpr int CH = 16 / (int)sizeof(T);
  constexpr int LDK = HD + CH, LDV = BKV + CH;           // padded LDS rows
  constexpr int NHB = HD / 16;                            // 16-row groups of the head dim
  typedef Mma<T> MM;
  constexpr int NKS = HD / MM::KSTEP;
  __shared__ __attribute__((aligned(16))) T sK[BKV * LDK];
  __shared__ __attribute__((aligned(16))) T sV[HD * LDV];
  __shared__ int sKp[BKV];

  const int b = blockIdx.y, kvh = blockIdx.z;
  const int qb = gridDim.x - 1 - blockIdx.x;             // longest blocks first
  const int nq = a.qcnt[b];
  if (qb * BQ >= nq) return;
  const int nk = a.kcnt[b];
  const int off = a.qmeta[1 + b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;

  const int qi = qb * BQ + wave * 16 + fr;                // this lane's query (index in sequence)
  const bool qvalid = qi < nq;
  const int myqpos = qvalid ? a.qpos[off + qi] : INT_MAX;
  const int wq0 = qb * BQ + wave * 16;
  const int wave_minpos = wq0 < nq ? a.qpos[off + wq0] : INT_MAX;
  const int qlast = min(qb * BQ + BQ - 1, nq - 1);
  const int maxpos = a.qpos[off + qlast];
  // keys visible to some query of this block: kpos <= maxpos (kpos ascending)
  const int* kp = a.kpos + (size_t)b * a.ldkpos;
  int lo = 0, hi = nk;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (kp[mid] <= maxpos) lo = mid + 1; else hi = mid;
  }
  const int kend = lo;

  const T* Qb = reinterpret_cast<const T*>(a.q);
  typename MM::frag qf[G][NKS];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (qvalid) {
        qf[hh][ks] = MM::load(Qb + (size_t)(off + qi) * a.ldq + (kvh * G + hh) * HD + ks * MM::KSTEP + g * MM::KW);
      } else {
        qf[hh][ks] = typename MM::frag{};
      }
    }

  float mrun[G], lrun[G];
  f32x4 o[G][NHB];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    mrun[hh] = -INFINITY;
    lrun[hh] = 0.f;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) o[hh][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const T* Kb = reinterpret_cast<const T*>(a.k) + (size_t)b * a.kpad * a.hkv * HD + kvh * HD;
  const T* Vb = reinterpret_cast<const T*>(a.vt) + ((size_t)b * a.hkv + kvh) * HD * a.kpad;
  const int ldk_g = a.hkv * HD;

  for (int t0 = 0; t0 < kend; t0 += BKV) {
    __syncthreads();
    // stage K rows [t0, t0+64) and V^T columns [t0, t0+64); tokens past nk read as zero
    for (int c = tid; c < BKV * (HD / CH); c += 256) {
      const int r = c / (HD / CH), cc = (c % (HD / CH)) * CH;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t0 + r < nk) v = *reinterpret_cast<const uint4*>(Kb + (size_t)(t0 + r) * ldk_g + cc);
      *reinterpret_cast<uint4*>(&sK[r * LDK + cc]) = v;
    }
    for (int c = tid; c < HD * (BKV / CH); c += 256) {
      const int r = c / (BKV / CH), cc = (c % (BKV / CH)) * CH;
      const T* src = Vb + (size_t)r * a.kpad + t0 + cc;
      T* dst = &sV[r * LDV + cc];
      if (t0 + cc + CH <= nk) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
#pragma unroll
        for (int e = 0; e < CH; ++e) dst[e] = (t0 + cc + e < nk) ? src[e] : from_f32<T>(0.f);
      }
    }
    if (tid < BKV) sKp[tid] = (t0 + tid < nk) ? kp[t0 + tid] : INT_MAX;
    __syncthreads();
    const bool need_mask = (t0 + BKV > nk) || (sKp[BKV - 1] > wave_minpos);

#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          typename MM::frag kf = MM::load(&sK[(kb * 16 + fr) * LDK + ks * MM::KSTEP + g * MM::KW]);
          s[kb] = MM::mma(kf, qf[hh][ks], s[kb]);
        }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = s[kb][e] * a.scale_log2;
          if (need_mask && sKp[kb * 16 + g * 4 + e] > myqpos) v = -INFINITY;
          s[kb][e] = v;
          mloc = fmaxf(mloc, v);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float mnew = fmaxf(mrun[hh], mloc);
      const float alpha = exp2f(mrun[hh] - mnew);
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float p = exp2f(s[kb][e] - mnew);
          s[kb][e] = p;
          lsum += p;
        }
      lrun[hh] = lrun[hh] * alpha + lsum;
      mrun[hh] = mnew;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) o[hh][hb] *= alpha;

      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          bf16x8 pf;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pf[e] = (bf16)s[2 * k2][e];
            pf[4 + e] = (bf16)s[2 * k2 + 1][e];
          }
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) {
            const T* vr = &sV[(hb * 16 + fr) * LDV + 32 * k2 + 4 * g];
            bf16x4 lo4 = *reinterpret_cast<const bf16x4*>(vr);
            bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(vr + 16);
            bf16x8 vf = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            o[hh][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[hh][hb], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) {
              const float vv = to_f32(sV[(hb * 16 + fr) * LDV + 16 * kb + 4 * g + e]);
              o[hh][hb] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, s[kb][e], o[hh][hb], 0, 0, 0);
            }
          }
      }
    }
  }

  if (!qvalid) return;
  T* Ob = reinterpret_cast<T*>(a.o) + (size_t)(off + qi) * a.ldo;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float l = lrun[hh];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.f / l;
    const int h = kvh * G + hh;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      Vec4<T>::store(Ob + h * HD + hb * 16 + 4 * g, o[hh][hb][0] * inv, o[hh][hb][1] * inv,
                     o[hh][hb][2] * inv, o[hh][hb][3] * inv);
  }
}

template <typename T, int HD>
static hipError_t launch_hd(const AttnArgs& a, dim3 grid, hipStream_t s) {
  const int G = a.hq / a.hkv;
  switch (G) {
    case 1: hipLaunchKernelGGL((k_attn<T, HD, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_attn<T, HD, 2>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_attn<T, HD, 3>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_attn<T, HD, 4>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attention(const AttnArgs& a, int B, int max_rows_per_seq, hipStream_t s) {
  dim3 grid((max_rows_per_seq + 63) / 64, B, a.hkv);
  if (grid.x == 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    if (a.hd == 64) return launch_attention_bf16(a, grid, s);
  } else {
    if (a.hd == 16) return launch_hd<T, 16>(a, grid, s);
    if (a.hd == 32) return launch_hd<T, 32>(a, grid, s);
    if (a.hd == 64) return launch_hd<T, 64>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_attention<float>(const AttnArgs&, int, int, hipStream_t);
template hipError_t launch_attention<bf16>(const AttnArgs&, int, int, hipStream_t);

}  // namespace mor
