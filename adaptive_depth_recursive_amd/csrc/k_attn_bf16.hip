// bf16 causal attention over per-recursion active sets (head_dim 64), tuned for gfx950.
//
// Same computation as the generic kernel in k_attn.hip (key s visible to query t iff
// kpos[s] <= qpos[t]; S^T = K Q^T on MFMA, online softmax per query column, P^T fed to the PV
// product as the B operand, V^T as the A operand), organised for throughput:
//  - K and V^T tiles of 64 keys, and their positions, stream global -> LDS with
//    global_load_lds (no register round trip) into two stages, so the next tile is in flight
//    while this one is used; the stages are separate LDS objects and the tile loop is unrolled
//    by two, which lets the compiler see that the reads of one stage do not wait for the
//    prefetch into the other;
//  - the K tile rows are read in a permuted key order, chosen so that the 8 keys a lane holds
//    for one PV step are 8 consecutive keys: the matching V^T operand is then one 16-byte LDS
//    read, and the S^T accumulators need no shuffles to become the P^T operand;
//  - K and V fragments are read once per tile and reused by all query heads of the KV head, and
//    the next head's S^T products are issued before this head's softmax (matrix cores and
//    vector ALUs overlap within a wave);
//  - the running maximum is only raised (and O rescaled) when it grows by more than 2^8, so the
//    rescale and its cross-lane reduction are skipped on most tiles; probabilities are then
//    bounded by 2^8, exact in fp32;
//  - workgroups are ordered so that each XCD owns whole (sequence, KV head) pairs, whose K/V then
//    stay in that XCD's L2, with query blocks longest first; the key range of a block is found
//    by a sampled wave-wide search while the first tile is already loading.
#include <climits>

#include "mor_internal.h"

namespace mor {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kRow = 128;                          // LDS row: 64 bf16

// V^T tile rows (head-dim index) are read 16 consecutive at a time: swizzle by (row >> 1) & 7.
__device__ __forceinline__ int swz_v(int row) { return (row >> 1) & 7; }
// K tile rows are read in the order perm(16h + 4a + b) = 8a + 4h + b within each 32 rows (see
// kslot); this swizzle gives those 16 rows 16 distinct bank groups.
__device__ __forceinline__ int swz_k(int row) { return (((row >> 3) & 3) << 1) | ((row >> 1) & 1); }

// LDS row of the K tile read by A-operand row `r` (0..63) of the S^T product.
__device__ __forceinline__ int kslot(int r) {
  const int blk = r & ~31, w = r & 31;
  const int h = w >> 4, a = (w >> 2) & 3, b = w & 3;
  return blk + 8 * a + 4 * h + b;
}

template <int ROWS>
__device__ __forceinline__ void dma_rows(const bf16* src, size_t ld, char* dst, int wave, int lane,
                                         bool kswz) {
  constexpr int INSTR = ROWS / 8 / 4;
#pragma unroll
  for (int i = 0; i < INSTR; ++i) {
    const int rb = (i * 4 + wave) * 8;
    const int r = rb + (lane >> 3);
    const int c = (lane & 7) ^ (kswz ? swz_k(r) : swz_v(r));
    __builtin_amdgcn_global_load_lds(src + (size_t)r * ld + c * 8, (lds_void*)(dst + rb * kRow), 16, 0, 0);
  }
}

// Maximum of finite-or-minus-infinity scores: v_max3 / v_max straight on the values (the
// compiler's fmaxf first quiets possible NaNs, which these scores never are).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ bf16x8 rd(const char* base, int row, int chunk, int sw) {
  return *reinterpret_cast<const bf16x8*>(base + row * kRow + ((chunk ^ sw) << 4));
}

}  // namespace

template <int G>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(AttnArgs a) {
  constexpr int BQ = 64, BKV = 64, HD = 64;
  constexpr int TILE = 2 * BKV * kRow;               // K tile + V^T tile
  // the two stages are separate LDS objects and the tile loop is unrolled by two, so the
  // compiler can tell the prefetch into one stage from the reads of the other and does not wait
  // for the prefetch before reading
  __shared__ __attribute__((aligned(1024))) char smem0[TILE];
  __shared__ __attribute__((aligned(1024))) char smem1[TILE];
  __shared__ int sKp0[BKV], sKp1[BKV];

  // Workgroups are dealt round-robin over the 8 XCDs by linear id. When the (sequence, KV head)
  // pairs split evenly over the XCDs, each XCD gets its own pairs (their K/V then stay in that
  // XCD's L2) and takes their query blocks longest first; otherwise the grid order is used.
  const int nqb = gridDim.x, npair = gridDim.y * gridDim.z;
  int b, kvh, qb;
  if (npair % 8 == 0) {
    const int lin = blockIdx.x + nqb * (blockIdx.y + gridDim.y * blockIdx.z);
    const int ppx = npair / 8, slot = lin >> 3;
    const int pair = (lin & 7) * ppx + slot % ppx;
    b = pair % gridDim.y;
    kvh = pair / gridDim.y;
    qb = nqb - 1 - slot / ppx;
  } else {
    b = blockIdx.y;
    kvh = blockIdx.z;
    qb = nqb - 1 - blockIdx.x;                       // longest blocks first
  }
  const int nq = a.qcnt[b];
  if (qb * BQ >= nq) return;
  const int nk = a.kcnt[b];
  const int off = a.qmeta[1 + b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;

  const int qi = qb * BQ + wave * 16 + fr;
  const bool qvalid = qi < nq;
  const int myqpos = qvalid ? a.qpos[off + qi] : INT_MAX;
  const int wq0 = qb * BQ + wave * 16;
  const int wave_minpos = wq0 < nq ? a.qpos[off + wq0] : INT_MAX;
  const int maxpos = a.qpos[off + min(qb * BQ + BQ - 1, nq - 1)];
  const int* kp = a.kpos + (size_t)b * a.ldkpos;
  const size_t ldk = (size_t)a.hkv * HD;
  const bf16* Kb = reinterpret_cast<const bf16*>(a.k) + (size_t)b * a.kpad * ldk + kvh * HD;
  const bf16* Vb = reinterpret_cast<const bf16*>(a.vt) + ((size_t)b * a.hkv + kvh) * HD * a.kpad;
  auto issue = [&](int t0, char* st, int* skp) {
    dma_rows<BKV>(Kb + (size_t)t0 * ldk, ldk, st, wave, lane, true);
    dma_rows<HD>(Vb + t0, a.kpad, st + BKV * kRow, wave, lane, false);
    // key positions go the same way (global -> LDS, no register round trip, so nothing waits on
    // them before the tile is needed); the index is clamped into the sequence, and keys at or
    // beyond nk are masked by index in the tile that holds them
    if (wave == 0)
      __builtin_amdgcn_global_load_lds(kp + min(t0 + lane, nk - 1), (lds_void*)skp, 4, 0, 0);
  };

  // Q fragments of the G heads, loaded once (the bf16 values the projection stored).
  const float sl2 = a.scale_log2;
  const bf16* Qb = reinterpret_cast<const bf16*>(a.q);
  bf16x8 qf[G][2];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      qf[hh][ks] = qvalid ? *reinterpret_cast<const bf16x8*>(Qb + (size_t)(off + qi) * a.ldq + (kvh * G + hh) * HD + ks * 32 + g * 8)
                          : bf16x8{};

  // Every query sees the first key tile, so its loads start before the key range is known.
  if (nk > 0) issue(0, smem0, sKp0);
  // kend = number of keys with position <= maxpos (positions ascend): each round samples the
  // remaining range at 64 evenly spaced keys, one per lane, and keeps the gap the count falls
  // in, so a few dependent loads replace a binary search's log2(nk)
  int lo = 0, hi = nk;
  while (hi - lo > 64) {
    const int stride = (hi - lo + 63) / 64;
    const int i = lo + lane * stride;
    const int c = __popcll(__ballot(i < hi && kp[i] <= maxpos));
    if (c == 0) { hi = lo; break; }
    hi = min(hi, lo + c * stride);
    lo += (c - 1) * stride + 1;
  }
  const int kend = lo + __popcll(__ballot(lo + lane < hi && kp[lo + lane] <= maxpos));

  // Per query (all four lanes that hold its column agree): reference maximum m of the scores in
  // base-2 units (score * scale * log2(e)), the running sum l of exp2(score * sl2 - m), and O.
  float mrun[G], lrun[G];
  f32x4 o[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    mrun[hh] = 0.f;
    lrun[hh] = 0.f;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) o[hh][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }



  const int ntiles = (kend + BKV - 1) / BKV;
  if (ntiles == 0 && nk > 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain tile 0
  // one key tile: wait for its stage, start the next tile's loads into the other stage, compute
  auto step = [&](int t, const char* sk, const int* kps, char* nst, int* nkp) {
    const int t0 = t * BKV;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < ntiles) issue(t0 + BKV, nst, nkp);
    const char* sv = sk + BKV * kRow;
    const bool need_mask = (t0 + BKV > nk) || (kps[BKV - 1] > wave_minpos);

    bf16x8 kf[4][2], vf[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int row = kslot(kb * 16 + fr);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) kf[kb][ks] = rd(sk, row, ks * 4 + g, swz_k(row));
    }
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int row = hb * 16 + fr;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) vf[hb][k2] = rd(sv, row, k2 * 4 + g, swz_v(row));
    }

    // positions of this lane's 16 keys, for the tiles that need the causal mask
    int kpv[4][4];
    if (need_mask) {
      const int lim = nk - t0 - 8 * g;                 // this lane's keys from index lim on are absent
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int4 p0 = *reinterpret_cast<const int4*>(&kps[32 * h2 + 8 * g]);
        const int4 p1 = *reinterpret_cast<const int4*>(&kps[32 * h2 + 8 * g + 4]);
        kpv[2 * h2][0] = p0.x; kpv[2 * h2][1] = p0.y; kpv[2 * h2][2] = p0.z; kpv[2 * h2][3] = p0.w;
        kpv[2 * h2 + 1][0] = p1.x; kpv[2 * h2 + 1][1] = p1.y; kpv[2 * h2 + 1][2] = p1.z; kpv[2 * h2 + 1][3] = p1.w;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (32 * h2 + 4 * hb + e >= lim) kpv[2 * h2 + hb][e] = INT_MAX;
      }
    }

    // S^T for one query head: the four key blocks are independent, so their first K halves are
    // issued before their second
    auto scores = [&](int hh, f32x4 (&s)[4]) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][0], qf[hh][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][1], qf[hh][1], s[kb], 0, 0, 0);
    };
    // Software pipeline over the query heads: the next head's S^T products are issued before
    // this head's softmax, so the matrix cores work while the vector ALUs do.
    f32x4 sc[4];
    scores(0, sc);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[kb] = sc[kb];
      if (hh + 1 < G) scores(hh + 1, sc);
      // s[kb][e]: raw score of key 32 (kb/2) + 8 g + 4 (kb & 1) + e of this tile
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kb][e] = kpv[kb][e] > myqpos ? -INFINITY : s[kb][e];
      }
      float mx = max3f(max3f(s[0][0], s[0][1], s[0][2]), max3f(s[0][3], s[1][0], s[1][1]),
                       max3f(s[1][2], s[1][3], s[2][0]));
      mx = max3f(mx, max3f(s[2][1], s[2][2], s[2][3]), max3f(s[3][0], s[3][1], s[3][2]));
      mx = max2f(mx, s[3][3]);
      // m is set on the first tile and afterwards raised (with O and l rescaled) only when a
      // score exceeds it by more than 2^8, so probabilities stay below 2^8 (exact in fp32); the
      // vote is wave-wide, the new m is agreed within each query's four lanes.
      if (t == 0 || __any(fmaf(mx, sl2, -mrun[hh]) > 8.f)) {
        mx = max2f(mx, __shfl_xor(mx, 16));
        mx = max2f(mx, __shfl_xor(mx, 32));
        const float mloc = mx * sl2;
        if (t == 0) {
          mrun[hh] = mloc;
        } else {
          const float mnew = fmaxf(mrun[hh], mloc);
          const float alpha = __builtin_amdgcn_exp2f(mrun[hh] - mnew);
          lrun[hh] *= alpha;
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) o[hh][hb] *= alpha;
          mrun[hh] = mnew;
        }
      }
      const float nm = -mrun[hh];
      float pr[4][4];
      bf16x8 pf[2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pr[kb][e] = __builtin_amdgcn_exp2f(fmaf(s[kb][e], sl2, nm));
          pf[kb >> 1][4 * (kb & 1) + e] = (bf16)pr[kb][e];
        }
      // the normaliser sums the unrounded probabilities, as a tree (short dependency chains)
      float ls[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) ls[kb] = (pr[kb][0] + pr[kb][1]) + (pr[kb][2] + pr[kb][3]);
      lrun[hh] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          o[hh][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[hb][k2], pf[k2], o[hh][hb], 0, 0, 0);
    }
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, smem0, sKp0, smem1, sKp1);
    if (t + 1 < ntiles) step(t + 1, smem1, sKp1, smem0, sKp0);
  }

  if (!qvalid) return;
  bf16* Ob = reinterpret_cast<bf16*>(a.o) + (size_t)(off + qi) * a.ldo;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float l = lrun[hh];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.f / l;
    const int h = kvh * G + hh;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      Vec4<bf16>::store(Ob + h * HD + hb * 16 + 4 * g, o[hh][hb][0] * inv, o[hh][hb][1] * inv,
                        o[hh][hb][2] * inv, o[hh][hb][3] * inv);
  }
}

hipError_t launch_attention_bf16(const AttnArgs& a, dim3 grid, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: hipLaunchKernelGGL((k_attn_bf16<1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_attn_bf16<2>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_attn_bf16<3>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_attn_bf16<4>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mor
