// bf16 projections of the Llama block on gfx950 MFMA, tiled for the CDNA4 CU.
//
// Same product and epilogues as the generic kernel in k_gemm.hip (C^T = W . A^T, weights on the
// MFMA A side, fp32 accumulation; QKV+RoPE+cache write, residual add, SwiGLU), organised for
// throughput:
//  - operand tiles move global -> LDS with global_load_lds_dwordx4 (no register staging): one
//    wave instruction writes 1 KB = 8 rows x 128 bytes of K, contiguous in LDS;
//  - LDS rows are 128 bytes (64 bf16 of K) with the 16-byte chunks XOR-swizzled by
//    (row >> 1) & 7, so the ds_read_b128 fragment reads of 16 consecutive rows hit 16 distinct
//    bank groups;
//  - 2 x NWM waves (4 or 8), each owning a (BN/2) x (BM/NWM) block of the output (BN weight
//    rows x BM activation rows per tile: four waves at 128 x 128, 192 x 128, 128 x 192 or 128 x 96
//    with two workgroups per CU, eight at 128 x 192 with two and at 256 x 256 with one); the
//    tile is chosen per launch from the number of rounds of resident workgroups it needs
//    (choose_tile below);
//  - two LDS stages: the loads of step k+1 are in flight while step k is multiplied;
//  - persistent workgroups (no more than are resident at once), each XCD owning a contiguous
//    range of the tile order so that the workgroups sharing an activation tile share its L2
//    (the hardware deals workgroups round-robin over the 8 XCDs); a workgroup issues its next
//    tile's first stage before the current tile's epilogue.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "mor_internal.h"

namespace mor {

namespace {

constexpr int kRowBytes = 128;                    // one LDS row: 64 bf16 of K
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Issue one stage's loads of NI wave instructions for one operand: with NW waves, instruction i
// moves the 8 rows starting at (NW i + wave) * 8, each lane its 16-byte chunk at element offset
// off[i] from `base`.
template <int NI, int NW>
__device__ __forceinline__ void load_stage(const bf16* base, const int* off, char* dst, int wave) {
#pragma unroll
  for (int i = 0; i < NI; ++i)
    __builtin_amdgcn_global_load_lds(base + off[i], (lds_void*)(dst + (i * NW + wave) * 8 * kRowBytes), 16, 0, 0);
}

__device__ __forceinline__ bf16x8 frag(const char* base, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(base + row * kRowBytes + ((chunk ^ swz(row)) << 4));
}

}  // namespace

template <int BN, int BM, int EPI, int NWM = 2>
__global__ __launch_bounds__(128 * NWM, (NWM == 4 && BN * BM <= 128 * 192) ? 2 : 1) void k_gemm_bf16(const bf16* __restrict__ A,
                                                      const bf16* __restrict__ W, int N, int K,
                                                      int tiles_n, int ntiles, int group_m,
                                                      const int* __restrict__ meta, GemmEpi ep) {
  constexpr int WN = BN / 2, WM = BM / NWM;
  constexpr int FN = WN / 16, FM = WM / 16;
  constexpr int STAGE = (BN + BM) * kRowBytes;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int M = meta[0];
  // Persistent workgroups: the grid holds at most as many workgroups as are resident at once,
  // and each takes a sequence of tiles. The hardware deals workgroups round-robin over the 8
  // XCDs (each with its own L2), so XCD x owns one contiguous range of the tile order and its
  // workgroups take that range's tiles in turn (round k of an XCD covers consecutive tiles).
  // The row count M is known only here (the host sizes the grid for its upper bound, e.g. under
  // token choice): only the row-blocks that hold rows are dealt out, so every XCD gets its share
  // of the real tiles.
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid % 8, slot = bid / 8;
  const int wpx = G / 8 + (xcd < G % 8 ? 1 : 0);            // workgroups on this XCD
  const int tiles_m = min(ntiles / tiles_n, (M + BM - 1) / BM);
  const int ntv = tiles_m * tiles_n;
  const int tpx = ntv / 8, trem = ntv % 8;
  const int tbase = xcd < trem ? xcd * (tpx + 1) : trem * (tpx + 1) + (xcd - trem) * tpx;
  const int tend = tbase + tpx + (xcd < trem ? 1 : 0);
  // Tile order: groups of group_m activation row-blocks, swept one weight column-block at a
  // time with the row-blocks fastest, so the workgroups resident on an XCD share a few
  // activation slabs and a few weight slabs in its L2.
  const int gsz = group_m * tiles_n;
  // the next tile of this workgroup at or after position t that has rows (m0 < M); -1 if none
  auto next_tile = [&](int t, int& m0, int& n0) -> int {
    for (; t < tend; t += wpx) {
      const int grp = t / gsz, gi = t - grp * gsz;
      const int rows_g = min(group_m, tiles_m - grp * group_m);
      const int tm = grp * group_m + gi % rows_g, tn = gi / rows_g;
      if (tm * BM < M) {
        m0 = tm * BM; n0 = tn * BN;
        return t;
      }
    }
    return -1;
  };
  int m0 = 0, n0 = 0;
  int t = next_tile(tbase + slot, m0, n0);
  if (t < 0) return;
  // clock sampling (measurement hook): the first workgroup, which always holds tile 0, reads the
  // shader cycle counter and the constant-rate real-time counter at its start and end
  const bool sample_clk = ep.clk != nullptr && bid == 0;
  long long clk_c0 = 0, clk_r0 = 0;
  if (sample_clk) { clk_c0 = clock64(); clk_r0 = wall_clock64(); }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave / NWM, wm = wave % NWM;
  const int fr = lane & 15, g = lane >> 4;

  f32x4 acc[FN][FM];

  // Operand tiles move global -> LDS with global_load_lds_dwordx4: one wave instruction writes
  // 1 KB = 8 rows x 128 bytes, contiguous in LDS; lane l loads the global 16-byte chunk that
  // lands at slot l & 7 of its row. The per-lane element offsets (from the tile's first row,
  // rows clamped into the operand) are computed once; a stage only adds its K offset.
  constexpr int NW = 2 * NWM;                     // waves: 2 along the weight rows x NWM
  constexpr int IW = BN / (8 * NW), IA = BM / (8 * NW);   // load instructions per wave per stage
  static_assert(IW * 8 * NW == BN && IA * 8 * NW == BM, "tile rows must split over the waves");
  const bf16* Wt;
  const bf16* At;
  int offw[IW], offa[IA];
  auto setup = [&](int tm0, int tn0) {
    Wt = W + (size_t)tn0 * K;
    At = A + (size_t)tm0 * K;
#pragma unroll
    for (int i = 0; i < IW; ++i) {
      const int r = (i * NW + wave) * 8 + (lane >> 3);
      offw[i] = min(r, N - 1 - tn0) * K + ((lane & 7) ^ swz(r)) * 8;
    }
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int r = (i * NW + wave) * 8 + (lane >> 3);
      offa[i] = min(r, M - 1 - tm0) * K + ((lane & 7) ^ swz(r)) * 8;
    }
  };
  auto issue = [&](int kt, int buf) {
    char* st = smem + buf * STAGE;
    load_stage<IW, NW>(Wt + kt * 64, offw, st, wave);
    load_stage<IA, NW>(At + kt * 64, offa, st + BN * kRowBytes, wave);
  };

  const int nk = K / 64;
  setup(m0, n0);
  issue(0, 0);
  int buf0 = 0;                                   // LDS stage of this tile's first K step
  for (;;) {
    const int g4 = g * 4;
    const int nw = n0 + wn * WN;
    const int mw = m0 + wm * WM + fr;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // residual epilogue of the 128 x 128 tile: the stream values this lane updates are loaded
    // during the last stage's matrix ops (no stage loads are in flight then), not after them
    constexpr bool kPrefetchX = EPI == EPI_RESID && BN * BM <= 128 * 128;
    float4 xr[kPrefetchX ? FN : 1][kPrefetchX ? FM : 1];

    for (int kt = 0; kt < nk; ++kt) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kt + 1 < nk) issue(kt + 1, (buf0 + kt + 1) & 1);
      if constexpr (kPrefetchX) {
        if (kt + 1 == nk) {
#pragma unroll
          for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int i = 0; i < FN; ++i) {
              const int m = mw + 16 * j, n = nw + 16 * i + g4;
              xr[i][j] = (m < M && n < N) ? *reinterpret_cast<const float4*>((ep.xin ? ep.xin : ep.x) + (size_t)m * ep.ldx + n)
                                          : float4{0.f, 0.f, 0.f, 0.f};
            }
        }
      }
      const char* sw = smem + ((buf0 + kt) & 1) * STAGE;
      const char* sa = sw + BN * kRowBytes;
      // both 32-deep halves' fragments are requested up front: the second half's reads are in
      // flight while the first half multiplies
      bf16x8 a[2][FN], b[2][FM];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < FN; ++i) a[ks][i] = frag(sw, wn * WN + i * 16 + fr, ks * 4 + g);
#pragma unroll
        for (int j = 0; j < FM; ++j) b[ks][j] = frag(sa, wm * WM + j * 16 + fr, ks * 4 + g);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks][i], b[ks][j], acc[i][j], 0, 0, 0);
      // keep that order through scheduling: the first half's reads, then its matrix ops with the
      // second half's reads spread between them, then the second half's matrix ops
      __builtin_amdgcn_sched_group_barrier(0x100, FN + FM, 0);
#pragma unroll
      for (int r = 0; r < FN + FM; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, FN * FM / (FN + FM), 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, FN * FM, 0);
    }

    // The next tile's first stage goes out before this tile's epilogue, into the stage the last
    // K step did not read (every wave passed the barrier after its last reads of it), so its
    // load latency overlaps the epilogue.
    int nm0 = 0, nn0 = 0;
    const int tnext = next_tile(t + wpx, nm0, nn0);
    if (tnext >= 0) {
      setup(nm0, nn0);
      issue(0, (buf0 + nk) & 1);
    }

    // ------------------------------------------------------------------ epilogues
    if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = mw + 16 * j;
        if (m >= M) continue;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int n = nw + 16 * i + g4;
          if (n >= N) continue;
          float4 v;
          if constexpr (kPrefetchX) v = xr[i][j];
          else v = *reinterpret_cast<const float4*>((ep.xin ? ep.xin : ep.x) + (size_t)m * ep.ldx + n);
          v.x += acc[i][j][0]; v.y += acc[i][j][1]; v.z += acc[i][j][2]; v.w += acc[i][j][3];
          *reinterpret_cast<float4*>(ep.x + (size_t)m * ep.ldx + n) = v;
        }
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = mw + 16 * j;
        if (m >= M) continue;
#pragma unroll
        for (int i = 0; i < FN; i += 2) {
          const int np = nw + 16 * i;
          if (np >= N) continue;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gt = acc[i][j][e], up = acc[i + 1][j][e];
            o[e] = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
          }
          Vec4<bf16>::store(reinterpret_cast<bf16*>(ep.h) + (size_t)m * ep.ldh + (np >> 1) + g4,
                            o[0], o[1], o[2], o[3]);
        }
      }
    } else {  // EPI_QKV, head_dim 64: the rotate-half partner of frag i is frag i + 2
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
          if (nf < ep.nq + ep.nkv) {
            if ((i & 3) >= 2) continue;               // second half: written with its partner
            const int rbase = nf < ep.nq ? 0 : ep.nq;
            const int c0 = (nf - rbase) & 63;         // 0 or 16
            float lo[4], hi[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int f = c0 + g4 + e;
              const float cs = ep.rope_cos[pos * 32 + f], sn = ep.rope_sin[pos * 32 + f];
              const float x1 = acc[i][j][e], x2 = acc[i + 2][j][e];
              lo[e] = x1 * cs - x2 * sn;
              hi[e] = x2 * cs + x1 * sn;
            }
            bf16* dst;
            if (nf < ep.nq) {
              dst = reinterpret_cast<bf16*>(ep.q) + (size_t)m * ep.ldq + nf + g4;
            } else {
              dst = reinterpret_cast<bf16*>(ep.k) + ((size_t)bseq * ep.kpad + bidx) * ep.nkv + (nf - ep.nq) + g4;
            }
            Vec4<bf16>::store(dst, lo[0], lo[1], lo[2], lo[3]);
            Vec4<bf16>::store(dst + 32, hi[0], hi[1], hi[2], hi[3]);
          } else {
            const int vn = nf - ep.nq - ep.nkv + g4;
            const int kvh = vn >> 6, dc = vn & 63;
            bf16* vp = reinterpret_cast<bf16*>(ep.vt) + (((size_t)bseq * ep.hkv + kvh) * 64 + dc) * ep.kpad + bidx;
#pragma unroll
            for (int e = 0; e < 4; ++e) vp[(size_t)e * ep.kpad] = (bf16)acc[i][j][e];
          }
        }
      }
    }
    if (tnext < 0) break;
    t = tnext; m0 = nm0; n0 = nn0;
    buf0 = (buf0 + nk) & 1;
  }
  if (sample_clk && threadIdx.x == 0) {
    atomicAdd(ep.clk, (unsigned long long)(clock64() - clk_c0));
    atomicAdd(ep.clk + 1, (unsigned long long)(wall_clock64() - clk_r0));
  }
}

namespace {

int g_group_m = -1;       // tuning override of the tile-order group (MOR_GEMM_GROUP_M)

// Workgroups of a launch: at most one per tile, and at most as many as are resident at once
// (256 CUs x per_cu), each then taking several tiles. Read at every launch: MOR_GEMM_PERSIST=0
// gives every tile its own workgroup (for measurement); MOR_GEMM_PERSIST=n caps the grid at n
// rounded up to a multiple of 8 (tests: many tiles per workgroup at small sizes). A grid smaller
// than the tile count is always a multiple of 8, so that every XCD owning tiles has workgroups.
int grid_size(int ntiles, int per_cu) {
  int cap = 256 * per_cu;
  if (const char* e = getenv("MOR_GEMM_PERSIST")) {
    const int v = atoi(e);
    if (v <= 0) return ntiles;
    cap = std::max(8, (v + 7) / 8 * 8);
  }
  return std::min(ntiles, cap);
}

int group_m() {
  if (g_group_m == -1) {
    g_group_m = 8;
    if (const char* s = getenv("MOR_GEMM_GROUP_M")) g_group_m = std::max(1, atoi(s));
  }
  return g_group_m;
}

// Tile override MOR_GEMM_TILE ("128x128", "192x128", "128x192", "128x96", "128x64", "256x128",
// "256x256", and the eight-wave "128x128w8", "128x192w8", "256x192w8", "192x256w8", "256x256w8");
// read at every launch (a getenv per projection), so a process can change it between calls.
int forced_tile() {
  const char* s = getenv("MOR_GEMM_TILE");
  if (!s) return 0;
  if (!strcmp(s, "256x256")) return 1;
  if (!strcmp(s, "256x128")) return 2;
  if (!strcmp(s, "128x128")) return 3;
  if (!strcmp(s, "192x128")) return 4;
  if (!strcmp(s, "128x192")) return 5;
  if (!strcmp(s, "128x96")) return 6;
  if (!strcmp(s, "128x64")) return 7;
  if (!strcmp(s, "256x192w8")) return 8;
  if (!strcmp(s, "192x256w8")) return 9;
  if (!strcmp(s, "256x256w8")) return 10;
  if (!strcmp(s, "128x192w8")) return 11;
  if (!strcmp(s, "128x128w8")) return 12;
  return 0;
}

template <int BN, int BM>
hipError_t launch_cfg(int epi, const bf16* A, const bf16* W, int N, int K, int m_upper,
                      const int* meta, const GemmEpi& ep, hipStream_t s) {
  const int tn = (N + BN - 1) / BN, tm = (m_upper + BM - 1) / BM;
  const int nblk = tn * tm;
  if (nblk == 0) return hipSuccess;
  const int gm = group_m();
  const dim3 grid(grid_size(nblk, BN * BM <= 128 * 192 ? 2 : 1));
  switch (epi) {
    case EPI_QKV: hipLaunchKernelGGL((k_gemm_bf16<BN, BM, EPI_QKV>), grid, dim3(256), 0, s, A, W, N, K, tn, nblk, gm, meta, ep); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemm_bf16<BN, BM, EPI_RESID>), grid, dim3(256), 0, s, A, W, N, K, tn, nblk, gm, meta, ep); break;
    default: hipLaunchKernelGGL((k_gemm_bf16<BN, BM, EPI_SWIGLU>), grid, dim3(256), 0, s, A, W, N, K, tn, nblk, gm, meta, ep); break;
  }
  return hipGetLastError();
}

// One epilogue only (tile shapes the QKV epilogue cannot use).
template <int BN, int BM, int EPI>
hipError_t launch_cfg_rs(const bf16* A, const bf16* W, int N, int K, int m_upper, const int* meta,
                         const GemmEpi& ep, hipStream_t s) {
  const int tn = (N + BN - 1) / BN, tm = (m_upper + BM - 1) / BM;
  const int nblk = tn * tm;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm_bf16<BN, BM, EPI>), dim3(grid_size(nblk, 2)), dim3(256), 0, s, A, W, N, K, tn, nblk, group_m(), meta, ep);
  return hipGetLastError();
}

// Eight waves (2 x 4) per workgroup, one workgroup per CU.
template <int BN, int BM>
hipError_t launch_cfg8(int epi, const bf16* A, const bf16* W, int N, int K, int m_upper,
                       const int* meta, const GemmEpi& ep, hipStream_t s) {
  const int tn = (N + BN - 1) / BN, tm = (m_upper + BM - 1) / BM;
  const int nblk = tn * tm;
  if (nblk == 0) return hipSuccess;
  const int gm = group_m();
  const dim3 grid(grid_size(nblk, BN * BM <= 128 * 192 ? 2 : 1));
  switch (epi) {
    case EPI_QKV: hipLaunchKernelGGL((k_gemm_bf16<BN, BM, EPI_QKV, 4>), grid, dim3(512), 0, s, A, W, N, K, tn, nblk, gm, meta, ep); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemm_bf16<BN, BM, EPI_RESID, 4>), grid, dim3(512), 0, s, A, W, N, K, tn, nblk, gm, meta, ep); break;
    default: hipLaunchKernelGGL((k_gemm_bf16<BN, BM, EPI_SWIGLU, 4>), grid, dim3(512), 0, s, A, W, N, K, tn, nblk, gm, meta, ep); break;
  }
  return hipGetLastError();
}

// Tile choice. A launch runs in rounds of as many tiles as fit on the chip at once (256 CUs x
// workgroups per CU); a round costs about the same whatever the tile count in it, so the
// estimate is rounds x the cost of one round of that tile relative to 128 x 128. Measured on
// the 360M-shape projections: a round of 192 x 128 or 128 x 192 tiles (1.5x the work) costs
// about 1.25 rounds of 128 x 128, the larger tiles reusing each LDS byte more; on a tie the
// taller activation tile (128 x 192) goes first, measured 1-3% faster than 192 x 128 there. A
// round of 128 x 96 tiles costs about 0.92 of a 128 x 128 round: it wins where 128 x 128 leaves
// a single round unevenly filled (the residual projections at a third of the tokens, 8% faster).
// A 256 x 256 tile of eight waves (one workgroup per CU) costs about 1.9 rounds of 128 x 128: it
// wins where 128 x 128 needs exactly two rounds (the residual projections at all 16,384 tokens,
// 77.3 -> 73.8 us). The four-wave 256-wide tiles, 128 x 64 and the other eight-wave shapes
// never won on these shapes and are left to MOR_GEMM_TILE.
struct TileCfg {
  int bn, bm, per_cu;
  double round_cost;
  int choice;       // forced_tile() value of the same tile
};
constexpr TileCfg kTiles[] = {{128, 128, 2, 1.0, 3}, {128, 192, 2, 1.25, 5}, {192, 128, 2, 1.25, 4},
                              {128, 96, 2, 0.92, 6}, {256, 256, 1, 1.9, 10}};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// rows_bound: m_upper only bounds the rows (they are counted on the device); a tile of one
// workgroup per CU would then leave most CUs idle when the real count is well below the bound,
// so only the two-per-CU tiles compete.
int choose_tile(int epi, int N, int m_upper, bool rows_bound) {
  int best = 0;
  double best_t = 1e300;
  for (int c = 0; c < kNumTiles; ++c) {
    if (kTiles[c].bn == 192 && epi == EPI_QKV) continue;   // the QKV epilogue needs 64-wide halves
    if (rows_bound && kTiles[c].per_cu < 2) continue;
    const long tiles = (long)((N + kTiles[c].bn - 1) / kTiles[c].bn) * ((m_upper + kTiles[c].bm - 1) / kTiles[c].bm);
    const long slots = 256L * kTiles[c].per_cu;
    const double t = (double)((tiles + slots - 1) / slots) * kTiles[c].round_cost;
    if (t < best_t - 1e-9) { best_t = t; best = c; }
  }
  return kTiles[best].choice;
}

}  // namespace

template <>
hipError_t launch_gemm<bf16>(int epi, const bf16* A, const bf16* W, int N, int K, int m_upper,
                             const int* meta, const GemmEpi& ep, hipStream_t s) {
  if (K % 64 || N % 64) return hipErrorInvalidValue;
  int choice = forced_tile();
  if (choice == 0) {
    choice = choose_tile(epi, N, m_upper, ep.rows_bound != 0);
    // 128 x 192 also runs as eight waves at two workgroups per CU (114 VGPRs, four waves per
    // SIMD): 2-6% faster for the QKV and residual epilogues, about 1% slower for SwiGLU
    if (choice == 5 && epi != EPI_SWIGLU) choice = 11;
  }
  // 192-wide weight tiles: residual and SwiGLU epilogues only (the QKV epilogue pairs the two
  // halves of a 64-wide head inside one wave's 64-column share)
  if (choice == 4 && epi == EPI_QKV) choice = 3;
  switch (choice) {
    case 1: return launch_cfg<256, 256>(epi, A, W, N, K, m_upper, meta, ep, s);
    case 2: return launch_cfg<256, 128>(epi, A, W, N, K, m_upper, meta, ep, s);
    case 4:
      if (epi == EPI_RESID) return launch_cfg_rs<192, 128, EPI_RESID>(A, W, N, K, m_upper, meta, ep, s);
      return launch_cfg_rs<192, 128, EPI_SWIGLU>(A, W, N, K, m_upper, meta, ep, s);
    case 5: return launch_cfg<128, 192>(epi, A, W, N, K, m_upper, meta, ep, s);
    case 6: return launch_cfg<128, 96>(epi, A, W, N, K, m_upper, meta, ep, s);
    case 7: return launch_cfg<128, 64>(epi, A, W, N, K, m_upper, meta, ep, s);
    case 8: return launch_cfg8<256, 192>(epi, A, W, N, K, m_upper, meta, ep, s);
    case 9:
      if (epi == EPI_QKV) return launch_cfg8<256, 192>(epi, A, W, N, K, m_upper, meta, ep, s);
      return launch_cfg8<192, 256>(epi, A, W, N, K, m_upper, meta, ep, s);
    case 10: return launch_cfg8<256, 256>(epi, A, W, N, K, m_upper, meta, ep, s);
    case 11: return launch_cfg8<128, 192>(epi, A, W, N, K, m_upper, meta, ep, s);
    case 12: return launch_cfg8<128, 128>(epi, A, W, N, K, m_upper, meta, ep, s);
    default: return launch_cfg<128, 128>(epi, A, W, N, K, m_upper, meta, ep, s);
  }
}

}  // namespace mor
