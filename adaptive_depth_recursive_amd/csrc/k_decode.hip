// Depth-wise batched MoR decode on gfx950 (reading notes section 4, continuous depth-wise
// batching; MoR paper A.3 and reading notes 3.1 / 3.2 for the per-recursion caches; reading notes
// 2.1 for the static sigmoid > 0.5 exit test used at inference).
//
// Every iteration advances each occupied slot by one recursion: a newly admitted token first runs
// the unique first layer, then every occupied slot runs the n_s shared layers at its own
// recursion depth (the tokens at different depths share the same weights, so they share every
// launch), then tokens whose next router logit is not positive -- or that reached N_r -- run the
// unique last layer and leave. A finished token's slot takes the request's next token, a finished
// request's slot takes the next request from the FIFO. All of this state lives on the device, so
// an iteration needs no host round trip.
//
// Slots are the rows of every decode GEMM (at most 64); rows whose slot takes no part in a layer
// are computed and ignored, so the launches have fixed grids.
//
// KV cache: pages of P tokens for one layer of one stream, K then V, each [hkv][P][hd]. Layer
// stream 0 = first layer, 1 = last layer, 2 + (r-1) n_s + (j-1) = shared layer j at recursion r.
// A page table per (slot, layer stream) maps the index of a cached token to its page. Pages come
// from a device free-list stack and return to it when the request finishes.
#include <algorithm>
#include <climits>

#include "mor_internal.h"

namespace mor {

namespace {

__device__ __forceinline__ int wave_scan_excl(int v, int* total) {
  const int lane = lane_id();
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  *total = __shfl(x, 63);
  return x - v;
}

__device__ __forceinline__ int layer_stream_shared(const DecArgs& a, int r, int j) {
  return 2 + (r - 1) * a.n_s + (j - 1);
}

typedef __attribute__((address_space(3))) void lds_void;

// Scheduling fences with no code: use_now makes a value (and so its load) complete here;
// opaque hides a value's origin, so arithmetic on it cannot be hoisted above this point.
__device__ __forceinline__ void use_now(int v) { asm volatile("" ::"s"(v)); }
__device__ __forceinline__ void use_now(long long v) { asm volatile("" ::"s"(v)); }
__device__ __forceinline__ void use_now(const void* v) { asm volatile("" ::"s"(v)); }
__device__ __forceinline__ void use_now(int a, int b, int c) { asm volatile("" ::"s"(a), "s"(b), "s"(c)); }
__device__ __forceinline__ void use_now(int a, int b, int c, int d, int e) {
  asm volatile("" ::"s"(a), "s"(b), "s"(c), "s"(d), "s"(e));
}
__device__ __forceinline__ void use_now(int a, int b, int c, int d, float e) {
  asm volatile("" ::"s"(a), "s"(b), "s"(c), "s"(d), "s"(e));
}
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Loads one field from each 64-byte line of the decode arguments together, so the kernel's
// later argument reads hit the scalar cache instead of each costing a round trip.
__device__ __forceinline__ void touch_args(const DecArgs& a) {
  asm volatile("" ::"s"(a.S), "s"(a.sl_req), "s"(a.ptab), "s"(a.X), "s"(a.px), "s"(a.stats));
}

// One 16-byte direct-to-LDS load per lane: lane l's 16 bytes land at dst + 16 l.
__device__ __forceinline__ void dma16(const uint4* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}
// The same with the non-temporal (streaming) cache policy, for K/V page reads: an iteration
// reads tens of MB of pages once each, which would otherwise push the layer weights (read every
// iteration) out of the caches.
__device__ __forceinline__ void dma16_nt(const uint4* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 2 /* nt */);
}

}  // namespace

// ------------------------------------------------------------------ scheduler (one wave)
// Lane s owns slot s. Order of work: finish the tokens that left last iteration (advance to the
// next position, or finish the request and return its pages), admit queued requests into free
// slots in slot order, then allocate the pages this iteration's KV appends need.
__global__ __launch_bounds__(64) void k_dec_schedule(DecArgs a) {
  const int s = lane_id();
  const bool valid = s < a.S;
  int* g = a.glob;
  if (g[G_HALT]) {
    if (valid) { a.sl_first[s] = 0; a.sl_part[s] = 0; a.sl_exit[s] = 0; }
    return;
  }
  const int nreq = g[G_NREQ];
  int req = valid ? a.sl_req[s] : -1;
  int pos = valid ? a.sl_pos[s] : 0;
  int depth = valid ? a.sl_depth[s] : 0;
  bool admit = false;
  int nfree = 0;
  bool finished = false;
  if (valid && req >= 0 && depth == 0) {
    if (pos + 1 < a.req_len[req]) {
      pos += 1;
      admit = true;
    } else {
      finished = true;
      const int len = a.sl_base[s] + a.req_len[req];
      nfree = 2 * ((len + a.P - 1) / a.P);
      for (int r = 1; r <= a.R; ++r)
        if (!a.kv_share || r == 1) nfree += a.n_s * ((a.sl_cnt[s * a.R + r - 1] + a.P - 1) / a.P);
    }
  }
  // return pages of finished requests (stack order: slot, layer stream, page index)
  int tot_free;
  const int top0 = g[G_TOP];
  int w = top0 + wave_scan_excl(nfree, &tot_free);
  if (finished) {
    for (int ls = 0; ls < a.LS; ++ls) {
      int n;
      if (ls < 2) {
        n = (a.sl_base[s] + a.req_len[req] + a.P - 1) / a.P;
      } else {
        const int r = (ls - 2) / a.n_s + 1;
        n = (a.kv_share && r > 1) ? 0 : (a.sl_cnt[s * a.R + r - 1] + a.P - 1) / a.P;
      }
      const int* pt = a.ptab + ((size_t)s * a.LS + ls) * a.pps;
      for (int i = 0; i < n; ++i) a.free_pages[w++] = pt[i];
    }
    req = -1;
  }
  // the pages just pushed may be popped below by other lanes: make the stores visible first
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  int top = top0 + tot_free;

  // admit queued requests into free slots, in slot order
  const bool isfree = valid && req < 0;
  int nfreeslots;
  const int rank = wave_scan_excl(isfree ? 1 : 0, &nfreeslots);
  const int next = g[G_NEXT];
  if (isfree && next + rank < nreq) {
    req = next + rank;
    pos = 0;
    admit = true;
    a.sl_base[s] = 0;
    for (int r = 0; r < a.R; ++r) a.sl_cnt[s * a.R + r] = 0;
  }
  const int taken = min(nfreeslots, max(0, nreq - next));

  const bool part = valid && req >= 0;
  const int r = admit ? 1 : depth;
  const int kpos = (part ? a.sl_base[s] : 0) + pos;   // cache index of the token in the unique layers
  int need = 0;
  bool need_u = false, need_s = false;
  if (part) {
    need_u = admit && (kpos % a.P == 0);
    need_s = (!a.kv_share || r == 1) && (a.sl_cnt[s * a.R + r - 1] % a.P == 0);
    need = (need_u ? 2 : 0) + (need_s ? a.n_s : 0);
  }
  int tot_need;
  int off = wave_scan_excl(need, &tot_need);
  const bool full = tot_need > top;
  if (!full && part) {
    int p = top - tot_need + off;
    if (need_u) {
      a.ptab[((size_t)s * a.LS + 0) * a.pps + kpos / a.P] = a.free_pages[p++];
      a.ptab[((size_t)s * a.LS + 1) * a.pps + kpos / a.P] = a.free_pages[p++];
    }
    if (need_s) {
      const int idx = a.sl_cnt[s * a.R + r - 1] / a.P;
      for (int j = 1; j <= a.n_s; ++j)
        a.ptab[((size_t)s * a.LS + layer_stream_shared(a, r, j)) * a.pps + idx] = a.free_pages[p++];
    }
  }
  if (valid) {
    a.sl_req[s] = req;
    a.sl_pos[s] = pos;
    a.sl_depth[s] = part ? r : 0;
    a.sl_first[s] = (!full && admit) ? 1 : 0;
    a.sl_part[s] = (!full && part) ? 1 : 0;
    a.sl_exit[s] = 0;
  }
  // algorithmic bytes of this iteration's first layer and shared block (the last layer's are
  // counted by k_dec_output once the exits are known)
  const long long kvtok = 2LL * a.hkv * a.hd * a.es;        // K and V of one token in one layer
  long long kv_rd = 0, kv_wr = 0, act = 0;
  int n_first = 0, n_part = 0;
  if (!full && part) {
    const int idx = a.sl_cnt[s * a.R + r - 1];
    if (admit) { kv_rd += (long long)kpos * kvtok; kv_wr += kvtok; act += 4LL * a.d; n_first = 1; }
    if (a.kv_share && r >= 2) {
      kv_rd += (long long)a.n_s * (a.sl_cnt[s * a.R] ) * kvtok;
    } else {
      kv_rd += (long long)a.n_s * idx * kvtok;
      kv_wr += (long long)a.n_s * kvtok;
    }
    n_part = 1;
  }
  int tot_first, tot_part;
  (void)wave_scan_excl(n_first, &tot_first);
  (void)wave_scan_excl(n_part, &tot_part);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kv_rd += __shfl_xor(kv_rd, o);
    kv_wr += __shfl_xor(kv_wr, o);
    act += __shfl_xor(act, o);
  }
  if (s == 0) {
    if (a.stats) {
      const long long wb = a.layer_weight_bytes * ((tot_first ? 1 : 0) + (tot_part ? a.n_s : 0));
      a.stats[ST_WEIGHT] += (unsigned long long)wb;
      a.stats[ST_KV_READ] += (unsigned long long)kv_rd;
      a.stats[ST_KV_WRITE] += (unsigned long long)kv_wr;
      a.stats[ST_ACT] += (unsigned long long)act;
    }
    g[G_NEXT] = next + taken;
    g[G_ITER] += 1;
    if (full) {
      g[G_HALT] = 1;
      g[G_TOP] = top;
      atomicOr(a.err, (unsigned)ERR_KV_FULL);
    } else {
      g[G_TOP] = top - tot_need;
      g[G_PEAK] = max(g[G_PEAK], a.kv_pages - (top - tot_need));
    }
  }
}

hipError_t launch_dec_schedule(const DecArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_dec_schedule, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

// Engine reset for a new set of requests: empty slots, full free-page stack, zero counters.
__global__ void k_dec_reset(DecArgs a, int n_req) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.kv_pages) a.free_pages[i] = a.kv_pages - 1 - i;
  if (i < a.S) {
    a.sl_req[i] = -1; a.sl_pos[i] = 0; a.sl_base[i] = 0; a.sl_depth[i] = 0;
    a.sl_first[i] = 0; a.sl_part[i] = 0; a.sl_exit[i] = 0;
    for (int r = 0; r < a.R; ++r) a.sl_cnt[i * a.R + r] = 0;
  }
  if (i < 64) a.gate[i] = 0.f;
  if (i < 64 * a.d) { a.X[i] = 0.f; a.Hs[i] = 0.f; }
  if (i < G_COUNT) a.glob[i] = (i == G_TOP) ? a.kv_pages : (i == G_NREQ) ? n_req : 0;
  if (a.stats && i < ST_COUNT) a.stats[i] = 0;
}

hipError_t launch_dec_reset(const DecArgs& a, int n_req, hipStream_t s) {
  const long n = std::max<long>(std::max<long>(a.kv_pages, 64L * a.d), G_COUNT);
  hipLaunchKernelGGL(k_dec_reset, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, n_req);
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm of the slot rows
// One 256-thread workgroup per slot row (thread t owns the float4 chunks t, t+256, ...). With
// gather_inputs (first layer), admitted slots first load their token's input hidden state into
// X, and every other row of X is cleared; with fold > 0 the residual projection's partial sums
// are first added into X (split order).
// Split-K partial sums are added to a value in split order, exactly as a plain loop would. The
// kMaxSplits loads are issued unconditionally and before the first add (splits past n re-read
// split 0, a valid address, and are not added), so a fold costs one memory round trip instead of
// one per split.
constexpr int kMaxSplits = 8;
template <typename V>
__device__ __forceinline__ V fold_splits(V v, const V* p, size_t stride, int n) {
  V pv[kMaxSplits];
#pragma unroll
  for (int q = 0; q < kMaxSplits; ++q) pv[q] = p[(q < n ? q : 0) * stride];
#pragma unroll
  for (int q = 0; q < kMaxSplits; ++q)
    if (q < n) v = v + pv[q];
  return v;
}

constexpr int ROW_THREADS = 256, ROW_CHUNKS = 4;   // rows up to 4096 elements

__device__ __forceinline__ float block_sum_fixed(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ float sq4(float4 v) { return v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w; }

// Last step of an RMSNorm of a row held as float4 chunks (thread t holds chunks t, t + 256, ...)
// with ss this thread's sum of squares: the workgroup sum, then out = v / rms * gain. Every
// kernel that normalises a slot row ends with this, so the sum is grouped the same way in each.
template <typename T>
__device__ __forceinline__ void row_norm_store(const float4* v, const float4* gg, float ss, int nc,
                                               int d, float eps, float* red, T* out) {
  ss = block_sum_fixed(ss, red);
  const float rinv = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int u = 0; u < ROW_CHUNKS; ++u) {
    const int c = threadIdx.x + u * ROW_THREADS;
    if (c < nc)
      Vec4<T>::store(out + 4 * c, v[u].x * rinv * gg[u].x, v[u].y * rinv * gg[u].y,
                     v[u].z * rinv * gg[u].z, v[u].w * rinv * gg[u].w);
  }
}

// RMSNorm of a slot row of X as it stands (rows of slots that a fused kernel does not update).
template <typename T>
__device__ __forceinline__ void norm_row_as_is(const float4* x, const float* gain, int nc, int d,
                                               float eps, float* red, T* out) {
  const float4* g4 = reinterpret_cast<const float4*>(gain);
  float4 v[ROW_CHUNKS], gg[ROW_CHUNKS];
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < ROW_CHUNKS; ++u) {
    const int c = threadIdx.x + u * ROW_THREADS;
    v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < nc) {
      gg[u] = g4[c];
      v[u] = x[c];
    }
    ss += sq4(v[u]);
  }
  row_norm_store<T>(v, gg, ss, nc, d, eps, red, out);
}

template <typename T, bool GATHER>
__global__ __launch_bounds__(ROW_THREADS) void k_dec_norm(DecArgs a, int fold, const float* __restrict__ g,
                                                          float eps, T* __restrict__ Xn) {
  __shared__ float red[4];
  touch_args(a);
  const int s = blockIdx.x, t = threadIdx.x;
  const int d = a.d, nc = d / 4;
  float4* x = reinterpret_cast<float4*>(a.X + (size_t)s * d);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  float4 v[ROW_CHUNKS], gg[ROW_CHUNKS];
  if (GATHER) {
    // the slot's flag, request and position in one round trip, then the request's row offset
    const int first = a.sl_first[s], req = a.sl_req[s], pos = a.sl_pos[s];
    use_now(first, req, pos);
    const float4* src = (first && req >= 0)
                            ? reinterpret_cast<const float4*>(a.inputs + (size_t)(a.req_off[req] + pos) * d)
                            : nullptr;
#pragma unroll
    for (int u = 0; u < ROW_CHUNKS; ++u) {
      const int c = t + u * ROW_THREADS;
      v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < nc) {
        if (src) v[u] = src[c];
        gg[u] = g4[c];
      }
    }
  } else {
    // the row, the partial sums and the gains all in one round trip
    const float4* px = reinterpret_cast<const float4*>(a.px + (size_t)s * d);
#pragma unroll
    for (int u = 0; u < ROW_CHUNKS; ++u) {
      const int c = t + u * ROW_THREADS;
      v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < nc) {
        gg[u] = g4[c];
        v[u] = fold_splits(x[c], px + c, (size_t)64 * d / 4, fold);
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < ROW_CHUNKS; ++u) {
    const int c = t + u * ROW_THREADS;
    if (c < nc && (GATHER || fold)) x[c] = v[u];
    ss += sq4(v[u]);
  }
  row_norm_store<T>(v, gg, ss, nc, d, eps, red, Xn + (size_t)s * d);
}

template <typename T>
hipError_t launch_dec_norm(const DecArgs& a, bool gather_inputs, int fold, const float* g,
                           float eps, T* Xn, hipStream_t s) {
  if (a.d > 4 * ROW_CHUNKS * ROW_THREADS || fold < 0 || fold > kMaxSplits) return hipErrorInvalidValue;
  if (gather_inputs)
    hipLaunchKernelGGL((k_dec_norm<T, true>), dim3(a.S), dim3(ROW_THREADS), 0, s, a, 0, g, eps, Xn);
  else
    hipLaunchKernelGGL((k_dec_norm<T, false>), dim3(a.S), dim3(ROW_THREADS), 0, s, a, fold, g, eps, Xn);
  return hipGetLastError();
}
template hipError_t launch_dec_norm<float>(const DecArgs&, bool, int, const float*, float, float*, hipStream_t);
template hipError_t launch_dec_norm<bf16>(const DecArgs&, bool, int, const float*, float, bf16*, hipStream_t);

// ------------------------------------------------------------------ recursion entry / exit
// Router logit of a row in the fixed order of k_router (lane l of 64 sums the products of
// elements l, l+64, ... in ascending order, product and sum rounded separately, then the pairwise
// fold): the products are formed by the whole workgroup into LDS, wave 0 runs the 64 chains.
__device__ __forceinline__ float row_logit_fixed(const float* prod, int d, float bias) {
  const int lane = threadIdx.x & 63;
  float p = 0.f;
  for (int i = lane; i < d; i += WAVE) p = add_rn(p, prod[i]);
  p = fold_fixed(p);
  p = add_rn(p, bias);
  return (p == 0.f) ? 0.f : p;
}

constexpr int ROW_MAX = 4 * ROW_CHUNKS * ROW_THREADS;

// Start of the recursion of every occupied slot: a newly admitted token's state is the first
// layer's output (plus its down projection's partial sums), a continuing token's state is
// carried in Hs; the shared block works on X. The gate of the recursion is
// sigmoid(theta_r . H + b_r). The first shared layer's RMSNorm of every slot row (gain, Xn) is
// done here too, saving its launch.
template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void k_dec_prep(DecArgs a, int fold, const float* __restrict__ gain,
                                                          float eps, T* __restrict__ Xn) {
  __shared__ float prod[ROW_MAX];
  __shared__ float red[4];
  touch_args(a);
  const int s = blockIdx.x, t = threadIdx.x;
  // the slot's state in one round trip, before the participation test
  const int part = a.sl_part[s], r = a.sl_depth[s], first = a.sl_first[s];
  const int req = a.sl_req[s], pos = a.sl_pos[s];
  use_now(part, r, first, req, pos);
  const int d = a.d, nc = d / 4;
  float4* __restrict__ x = reinterpret_cast<float4*>(a.X + (size_t)s * d);
  T* out = Xn + (size_t)s * d;
  if (!part) {
    norm_row_as_is<T>(x, gain, nc, d, eps, red, out);
    return;
  }
  float4* __restrict__ hs = reinterpret_cast<float4*>(a.Hs + (size_t)s * d);
  const float4* __restrict__ w = reinterpret_cast<const float4*>(a.router_w + (size_t)(r - 1) * d);
  const float4* __restrict__ px = reinterpret_cast<const float4*>(a.px + (size_t)s * d);
  const float4* g4 = reinterpret_cast<const float4*>(gain);
  // the request's row offset and the router bias are only needed at the end: read now, used late
  const int roff = a.req_off[req];
  const float bias = a.router_b[r - 1];
  // all loads first (both the folded first-layer output and the carried state, so no branch
  // separates them), then the stores (a store to x or hs would order later loads behind it)
  float4 h[ROW_CHUNKS], wv[ROW_CHUNKS], gg[ROW_CHUNKS];
#pragma unroll
  for (int u = 0; u < ROW_CHUNKS; ++u) {
    const int c = t + u * ROW_THREADS;
    h[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < nc) {
      wv[u] = w[c];
      gg[u] = g4[c];
      const float4 hv = hs[c];
      const float4 fv = fold_splits(x[c], px + c, (size_t)64 * d / 4, fold);
      // component-wise: a select of whole float4 values is turned into an indexed private array
      h[u] = make_float4(first ? fv.x : hv.x, first ? fv.y : hv.y, first ? fv.z : hv.z,
                         first ? fv.w : hv.w);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < ROW_CHUNKS; ++u) {
    const int c = t + u * ROW_THREADS;
    if (c < nc) {
      if (first) hs[c] = h[u];             // the folded first-layer output is the state...
      x[c] = h[u];                         // ...and the shared block's input
      prod[4 * c + 0] = mul_rn(h[u].x, wv[u].x);
      prod[4 * c + 1] = mul_rn(h[u].y, wv[u].y);
      prod[4 * c + 2] = mul_rn(h[u].z, wv[u].z);
      prod[4 * c + 3] = mul_rn(h[u].w, wv[u].w);
    }
    ss += sq4(h[u]);
  }
  row_norm_store<T>(h, gg, ss, nc, d, eps, red, out);   // its barriers also publish prod
  const int tok = opaque(roff) + pos;
  if (first && a.h_dump) {
    float4* dump = reinterpret_cast<float4*>(a.h_dump + ((size_t)tok * (a.R + 1)) * d);
#pragma unroll
    for (int u = 0; u < ROW_CHUNKS; ++u) {
      const int c = t + u * ROW_THREADS;
      if (c < nc) dump[c] = h[u];
    }
  }
  if (t >= WAVE) return;
  const float z = row_logit_fixed(prod, d, bias);
  if (t == 0) {
    if (z != z) atomicOr(a.err, (unsigned)ERR_NAN_LOGIT);
    a.gate[s] = a.unit_gate ? -1.f : 1.f / (1.f + __expf(-z));
    if (a.z_dump) a.z_dump[(size_t)tok * a.R + (r - 1)] = z;
  }
}

template <typename T>
hipError_t launch_dec_prep(const DecArgs& a, int fold, const float* gain, float eps, T* Xn, hipStream_t s) {
  if (fold < 0 || fold > kMaxSplits) return hipErrorInvalidValue;
  if (a.d > ROW_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_dec_prep<T>), dim3(a.S), dim3(ROW_THREADS), 0, s, a, fold, gain, eps, Xn);
  return hipGetLastError();
}
template hipError_t launch_dec_prep<float>(const DecArgs&, int, const float*, float, float*, hipStream_t);
template hipError_t launch_dec_prep<bf16>(const DecArgs&, int, const float*, float, bf16*, hipStream_t);

__device__ __forceinline__ float gate_mix(float g, float xv, float hv) {
  return (g < 0.f) ? xv : hv + g * (xv - hv);
}

// End of the recursion: F(H) = X + the last shared layer's down-projection partial sums;
// H <- H + g (F(H) - H) (or F(H) under unit gating), then the exit test on the next router
// logit: the token continues iff r < N_r and theta_{r+1} . H + b_{r+1} > 0. The last layer's
// RMSNorm of every slot row (gain, Xn) is done here too, saving its launch.
template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void k_dec_update(DecArgs a, int fold, const float* __restrict__ gain,
                                                            float eps, T* __restrict__ Xn) {
  __shared__ float prod[ROW_MAX];
  __shared__ float red[4];
  touch_args(a);
  const int s = blockIdx.x, t = threadIdx.x;
  // the slot's state in one round trip, before the participation test
  const int part = a.sl_part[s], r = a.sl_depth[s], req = a.sl_req[s], pos = a.sl_pos[s];
  const float g = a.gate[s];
  use_now(part, r, req, pos, g);
  const int d = a.d, nc = d / 4;
  float4* __restrict__ x = reinterpret_cast<float4*>(a.X + (size_t)s * d);
  T* out = Xn + (size_t)s * d;
  if (!part) {
    norm_row_as_is<T>(x, gain, nc, d, eps, red, out);
    return;
  }
  float4* __restrict__ hs = reinterpret_cast<float4*>(a.Hs + (size_t)s * d);
  const float4* __restrict__ px = reinterpret_cast<const float4*>(a.px + (size_t)s * d);
  const float4* g4 = reinterpret_cast<const float4*>(gain);
  // the next recursion's router row (a valid row even after the last recursion, unused there),
  // and what is only needed at the end (row offset, bias, recursion count): read now, used late
  const bool next = r < a.R;
  const float4* __restrict__ w =
      reinterpret_cast<const float4*>(a.router_w + (size_t)min(r, a.R - 1) * d);
  const int roff = a.req_off[req];
  const float bias = a.router_b[min(r, a.R - 1)];
  const int done_r = a.sl_cnt[s * a.R + r - 1];
  // all loads first, then the stores
  float4 hn[ROW_CHUNKS], wv[ROW_CHUNKS], gg[ROW_CHUNKS];
#pragma unroll
  for (int u = 0; u < ROW_CHUNKS; ++u) {
    const int c = t + u * ROW_THREADS;
    hn[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < nc) {
      gg[u] = g4[c];
      wv[u] = w[c];
      const float4 hv = hs[c];
      const float4 xv = fold_splits(x[c], px + c, (size_t)64 * d / 4, fold);
      hn[u] = make_float4(gate_mix(g, xv.x, hv.x), gate_mix(g, xv.y, hv.y), gate_mix(g, xv.z, hv.z),
                          gate_mix(g, xv.w, hv.w));
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < ROW_CHUNKS; ++u) {
    const int c = t + u * ROW_THREADS;
    if (c < nc) {
      hs[c] = hn[u];
      x[c] = hn[u];
      if (next) {
        prod[4 * c + 0] = mul_rn(hn[u].x, wv[u].x);
        prod[4 * c + 1] = mul_rn(hn[u].y, wv[u].y);
        prod[4 * c + 2] = mul_rn(hn[u].z, wv[u].z);
        prod[4 * c + 3] = mul_rn(hn[u].w, wv[u].w);
      }
    }
    ss += sq4(hn[u]);
  }
  row_norm_store<T>(hn, gg, ss, nc, d, eps, red, out);  // its barriers also publish prod
  const int tok = opaque(roff) + pos;
  if (a.h_dump) {
    float4* dump = reinterpret_cast<float4*>(a.h_dump + ((size_t)tok * (a.R + 1) + r) * d);
#pragma unroll
    for (int u = 0; u < ROW_CHUNKS; ++u) {
      const int c = t + u * ROW_THREADS;
      if (c < nc) dump[c] = hn[u];
    }
  }
  if (t >= WAVE) return;
  bool leave = true;
  if (next) {
    const float p = row_logit_fixed(prod, d, bias);
    leave = !(p > 0.f);
    if (t == 0) {
      if (p != p) atomicOr(a.err, (unsigned)ERR_NAN_LOGIT);
      if (a.z_dump) a.z_dump[(size_t)tok * a.R + r] = p;
    }
  }
  if (t == 0) {
    a.sl_cnt[s * a.R + r - 1] = done_r + 1;
    if (leave) {
      a.sl_exit[s] = 1;
      a.exit_depth[tok] = (signed char)r;
    } else {
      a.sl_depth[s] = r + 1;
    }
  }
}

template <typename T>
hipError_t launch_dec_update(const DecArgs& a, int fold, const float* gain, float eps, T* Xn, hipStream_t s) {
  if (fold < 0 || fold > kMaxSplits) return hipErrorInvalidValue;
  if (a.d > ROW_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_dec_update<T>), dim3(a.S), dim3(ROW_THREADS), 0, s, a, fold, gain, eps, Xn);
  return hipGetLastError();
}
template hipError_t launch_dec_update<float>(const DecArgs&, int, const float*, float, float*, hipStream_t);
template hipError_t launch_dec_update<bf16>(const DecArgs&, int, const float*, float, bf16*, hipStream_t);

// Tokens that ran the last layer: output = X + the last layer's down-projection partial sums;
// mark the token finished. Workgroup 0 also counts the last layer's algorithmic bytes.
__global__ __launch_bounds__(ROW_THREADS) void k_dec_output(DecArgs a, int fold) {
  const int s = blockIdx.x, t = threadIdx.x;
  if (a.stats && s == 0 && t < 64) {
    // last-layer bytes of this iteration (every slot's exit flag is still set here)
    const long long kvtok = 2LL * a.hkv * a.hd * a.es;
    const bool ex = t < a.S && a.sl_exit[t];
    long long rd = ex ? (long long)(a.sl_base[t] + a.sl_pos[t]) * kvtok : 0;
    int n = ex ? 1 : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      rd += __shfl_xor(rd, o);
      n += __shfl_xor(n, o);
    }
    if (t == 0 && n) {
      a.stats[ST_WEIGHT] += (unsigned long long)a.layer_weight_bytes;
      a.stats[ST_KV_READ] += (unsigned long long)rd;
      a.stats[ST_KV_WRITE] += (unsigned long long)(n * kvtok);
      a.stats[ST_ACT] += (unsigned long long)(n * 4LL * a.d);
    }
  }
  __syncthreads();
  if (!a.sl_exit[s]) return;
  const int d = a.d;
  const int tok = a.req_off[a.sl_req[s]] + a.sl_pos[s];
  const float4* x = reinterpret_cast<const float4*>(a.X + (size_t)s * d);
  float4* o = reinterpret_cast<float4*>(a.outputs + (size_t)tok * d);
  for (int c = t; c < d / 4; c += ROW_THREADS) {
    o[c] = fold_splits(x[c], reinterpret_cast<const float4*>(a.px + (size_t)s * d) + c,
                       (size_t)64 * d / 4, fold);
  }
  if (t == 0) {
    a.sl_depth[s] = 0;                     // the exit flag is cleared by the next schedule
    atomicAdd(&a.glob[G_TOKENS], 1);
    if (a.sl_pos[s] + 1 == a.req_len[a.sl_req[s]]) atomicAdd(&a.glob[G_REQS], 1);
  }
}

hipError_t launch_dec_output(const DecArgs& a, int fold, hipStream_t s) {
  if (fold < 0 || fold > kMaxSplits) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_dec_output, dim3(a.S), dim3(ROW_THREADS), 0, s, a, fold);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decode attention
// One workgroup per (slot, KV head). It rotates the slot's new query heads and key (RoPE at the
// token's position, fp32, then rounded to the element type), appends the new K/V to the slot's
// page of the layer stream, and attends over the cached keys of that stream plus the new one:
// recursion-wise caching reads the stream of the token's own recursion; recursive KV sharing at
// r >= 2 appends nothing and reads the recursion-1 stream of the same shared layer.
// A page holds one layer stream's K as [hkv][P][hd] and V transposed as [hkv][hd][P], so that
// both operands of the products are contiguous along their reduction index: K along the head
// dimension (scores), V^T along the keys (probabilities x values).
// Waves take 64-key tiles in turn (wave w: keys 64 w, 64 (w + NW), ...); each keeps its own
// running maximum, normaliser and output, and the waves' partial results (plus the new key's,
// kept apart) are merged in a fixed order.
//  - bf16: both products on MFMA. S^T = K Q^T with the keys as rows, read in a permuted order
//    so that the scores a lane holds are, head by head, the 8 consecutive keys it supplies to
//    the P V product (P as the A operand, V^T fragments straight from the page): no shuffles
//    between the two products, no LDS for K or V.
//  - fp32: lane = key for the scores (its K row in registers), lane = head-dim element for the
//    values (its V^T row of the tile in registers).

// Waves per (slot, KV head) workgroup: 16 for bf16 (64-key tiles on MFMA, registers for both
// operand tiles), 8 for fp32; a context of n keys takes ceil(n / (64 NW)) tiles per wave.
#ifndef MOR_DEC_ATTN_WAVES_BF16
#define MOR_DEC_ATTN_WAVES_BF16 16
#endif
template <typename T, int HD, int G> constexpr int dec_attn_waves() {
  return sizeof(T) == 2 ? MOR_DEC_ATTN_WAVES_BF16 : 8;
}

// Page of key index k of a layer stream, and the element offset of its K row / V^T column.
__device__ __forceinline__ int dec_page(const int* pt, int k, int P) { return pt[k / P]; }

template <typename T, int HD, int G, int NW = dec_attn_waves<T, HD, G>()>
__global__ __launch_bounds__(NW * 64) void k_dec_attn(DecArgs a, int kind, int j) {
  constexpr int KT = 64;
  constexpr bool MF = sizeof(T) == 2;                // bf16: MFMA tile products
  static_assert(!MF || (HD == 64 && G <= 4), "bf16 decode attention: head dim 64, at most 4 query heads per KV head");
  __shared__ float sq[G][HD];
  __shared__ float skn[HD], svn[HD];
  __shared__ float sp[MF ? 1 : NW][G][KT];
  __shared__ float sm[NW + 1][G], sl[NW + 1][G];
  __shared__ float sacc[NW + 1][G][HD];
  // bf16: each wave's V^T tile [64 head-dim rows][64 keys], 128-byte rows with the 16-byte
  // chunks XOR-swizzled by (row / 2) % 8 (the fragment reads of 16 consecutive rows then hit
  // distinct bank groups)
  __shared__ __attribute__((aligned(16))) T svt[MF ? NW : 1][MF ? KT * HD : 1];

  touch_args(a);
  const int s = blockIdx.x, kvh = blockIdx.y;       // the grid has one row per slot
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = a.P;
  // The page numbers of this wave's first tile (keys 64 w .. 64 w + 63, at most 4 pages) are
  // read before the slot's depth is known, for every layer stream the depth could select (the
  // unique layer's stream, or recursion c + 1's stream of shared position j): lane 4 c + i
  // holds page i of candidate c. Entries past a stream's allocated pages are still valid page
  // numbers (the table is cleared at init and only ever holds page numbers), and the keys they
  // would serve are masked.
  const int ncand = kind == DL_SHARED ? a.R : 1;
  int spec_pg = 0;
  {
    const int c = lane >> 2, i = lane & 3;
    if (c < ncand) {
      const int ls = kind == DL_FIRST ? 0 : kind == DL_LAST ? 1 : layer_stream_shared(a, c + 1, j);
      spec_pg = a.ptab[((size_t)s * a.LS + ls) * a.pps + min(wave * KT / P + i, a.pps - 1)];
    }
  }
  // The slot's state in the same round trip: flag, position, depth and every per-recursion
  // count (the count this layer needs depends on the depth). The empty asm uses every value
  // before the participation test, so the compiler cannot move the other loads behind it.
  const int* flag = kind == DL_FIRST ? a.sl_first : kind == DL_LAST ? a.sl_exit : a.sl_part;
  const int part = flag[s];
  const int sbase = a.sl_base[s], spos = a.sl_pos[s], r = a.sl_depth[s];
  int cnt[MOR_MAX_REC_DEV];
#pragma unroll
  for (int q = 0; q < MOR_MAX_REC_DEV; ++q) cnt[q] = a.sl_cnt[s * a.R + min(q, a.R - 1)];
  use_now(part); use_now(sbase); use_now(spos); use_now(r);
#pragma unroll
  for (int q = 0; q < MOR_MAX_REC_DEV; ++q) use_now(cnt[q]);
  asm volatile("" ::"v"(spec_pg));
  // the arguments used before the first barrier, so their loads share the first round trip
  use_now(a.n_s); use_now(a.P); use_now(a.pps); use_now(a.LS); use_now(a.nqkv); use_now(a.kv_share);
  use_now(a.page_elems); use_now(a.ptab); use_now(a.pool); use_now(a.qkv); use_now(a.rope_cos);
  use_now(a.kqkv);
  if (!part) return;
  const int pos = sbase + spos;                      // position in the sequence
  int ls_w, ls_r, idx_w, nkeys;
  if (kind == DL_FIRST || kind == DL_LAST) {
    ls_w = ls_r = (kind == DL_FIRST) ? 0 : 1;
    idx_w = pos;
    nkeys = pos;
  } else if (a.kv_share && r >= 2) {
    ls_w = -1;
    ls_r = layer_stream_shared(a, 1, j);
    idx_w = 0;
    nkeys = cnt[0];
  } else {
    ls_w = ls_r = layer_stream_shared(a, r, j);
    int c = cnt[0];
#pragma unroll
    for (int q = 1; q < MOR_MAX_REC_DEV; ++q)
      if (q == r - 1) c = cnt[q];
    idx_w = c;
    nkeys = c;
  }
  T* pool = reinterpret_cast<T*>(a.pool);
  const size_t vofs = (size_t)a.hkv * P * HD;        // V^T part of a page
  // candidate of the stream read here: recursion r's (shared, recursion-wise), recursion 1's
  // (shared under KV sharing), the unique layer's
  const int csel = (kind == DL_SHARED && !(a.kv_share && r >= 2)) ? r - 1 : 0;
  const int* pt = a.ptab + ((size_t)s * a.LS + ls_r) * a.pps;
  // page of the appended key and value, read early by the threads that store them (a per-thread
  // value, so nothing waits for it before the barrier)
  const int page_w = (ls_w >= 0 && tid < 2 * HD) ? a.ptab[((size_t)s * a.LS + ls_w) * a.pps + idx_w / P] : 0;
  const int fr = lane & 15, g = lane >> 4;

  // This wave's first tile is issued before the query/key/value fold below, so its page-table
  // and row loads overlap the fold's.
  //  K/V page reads use the non-temporal cache policy (see dma16_nt).
  //  bf16: K fragments kf[kb][ks] into registers (A operand of S^T: row fr of key block kb is
  //  the key t0 + 32 (kb / 2) + 8 (fr / 4) + 4 (kb % 2) + fr % 4, head-dim elements
  //  32 ks + 8 g ..+7), and the V^T tile into the wave's LDS tile by direct-to-LDS loads
  //  (instruction q, lane l: LDS chunk 64 q + l = row (64 q + l) / 8, physical chunk l % 8,
  //  i.e. keys 8 ((l % 8) ^ swizzle(row)) ..+7 of that head-dim row). Keys past the context
  //  read the last cached key (valid memory; an 8-key group never crosses a page: P is a
  //  multiple of 8); their scores are masked (zero probabilities).
  //  fp32: lane = key: its K row; lane = head-dim element: its V^T row of the tile.
  int t0 = wave * KT;
  const bool lane_c = lane < HD;
  bf16x8 kf[MF ? 4 : 1][2];
  constexpr int KCH = MF ? 1 : HD / 4;               // fp32: 16-byte chunks of a K row
  float4 kr32[KCH], vr32[MF ? 1 : KT / 4];
  // page of key k of tile tt: on the wave's first tile from the speculative reads (a lane
  // exchange), on later tiles from the page table
  auto page_of = [&](int tt, int k, bool first) -> int {
    return first ? __shfl(spec_pg, 4 * csel + (k / P - tt / P)) : dec_page(pt, k, P);
  };
  auto issue_tile = [&](int tt, bool first) {
    if constexpr (MF) {
      // every page number in hand before the first row load (the compiler's wait for a
      // register loaded before a direct-to-LDS load is a full drain, which would serialise them)
      int kpg[4], vpg[8];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key = min(tt + 32 * (kb >> 1) + 8 * (fr >> 2) + 4 * (kb & 1) + (fr & 3), nkeys - 1);
        kpg[kb] = opaque(page_of(tt, key, first));
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = (64 * q + lane) >> 3;
        const int key = min(tt + 8 * ((lane & 7) ^ ((row >> 1) & 7)), (nkeys - 1) & ~7);
        vpg[q] = opaque(page_of(tt, key, first));
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key = min(tt + 32 * (kb >> 1) + 8 * (fr >> 2) + 4 * (kb & 1) + (fr & 3), nkeys - 1);
        const T* kp = pool + (size_t)kpg[kb] * a.page_elems + ((size_t)kvh * P + key % P) * HD;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          kf[kb][ks] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(kp + 32 * ks + 8 * g));
      }
      char* dst = reinterpret_cast<char*>(svt[wave]);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = (64 * q + lane) >> 3;
        const int key = min(tt + 8 * ((lane & 7) ^ ((row >> 1) & 7)), (nkeys - 1) & ~7);
        const T* vp = pool + (size_t)vpg[q] * a.page_elems + vofs + ((size_t)kvh * HD + row) * P + key % P;
        dma16_nt(reinterpret_cast<const uint4*>(vp), dst + q * 1024);
      }
    } else {
      const int key = min(tt + lane, nkeys - 1);
      const T* kp = pool + (size_t)page_of(tt, key, first) * a.page_elems + ((size_t)kvh * P + key % P) * HD;
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kp + 4 * c));
        kr32[c] = make_float4(v[0], v[1], v[2], v[3]);
      }
#pragma unroll
      for (int q = 0; q < KT / 4; ++q) {
        const int k4 = min(tt + 4 * q, (nkeys - 1) & ~3);
        const int pg = page_of(tt, k4, first);      // a lane exchange: every lane takes part
        if (lane_c) {
          const T* vp = pool + (size_t)pg * a.page_elems + vofs + ((size_t)kvh * HD + lane) * P + k4 % P;
          const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vp));
          vr32[q] = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  };
  // Query heads, key and value of the slot's token: the K-split partial sums added in split
  // order, RoPE on q and k, rounded to the element type. Thread i < (G + 2) HD owns element i
  // (the grid has at least that many threads): its loads (both halves' partial sums and the
  // rotation) are issued first, then this wave's first K/V tile, then the fold, which therefore
  // waits only for its own loads.
  static_assert(NW * 64 >= (G + 2) * HD, "one fold element per thread");
  const int half = HD / 2;
  const bool fold_on = tid < (G + 2) * HD;
  const int fh = tid / HD, fc = tid % HD;
  const int fpc = fc < half ? fc + half : fc - half;
  float f0[kMaxQkvSplits], f1[kMaxQkvSplits], fcs = 0.f, fsn = 0.f;
  {
    const float* qkv = a.qkv + (size_t)s * a.nqkv;
    const float* base = fh < G ? qkv + (kvh * G + min(fh, G - 1)) * HD
                        : fh == G ? qkv + a.nq + kvh * HD : qkv + a.nq + a.nkv + kvh * HD;
    const size_t split = (size_t)64 * a.nqkv;       // partial sums of the K splits
    const int nsp = a.kqkv;
    if (fold_on) {
      const int f = fc % half;
      fcs = a.rope_cos[pos * half + f];
      fsn = a.rope_sin[pos * half + f];
#pragma unroll
      for (int q = 0; q < kMaxQkvSplits; ++q) {     // splits past nsp re-read split 0 (unused)
        f0[q] = base[(q < nsp ? q : 0) * split + fc];
        f1[q] = base[(q < nsp ? q : 0) * split + fpc];
      }
    }
  }
  if (t0 < nkeys) issue_tile(t0, true);
  if (fold_on) {
    float v0 = f0[0], vp = f1[0];
#pragma unroll
    for (int q = 1; q < kMaxQkvSplits; ++q)
      if (q < a.kqkv) { v0 = v0 + f0[q]; vp = vp + f1[q]; }
    const float rot = fc < half ? v0 * fcs - vp * fsn : v0 * fcs + vp * fsn;
    const float v = to_f32(from_f32<T>(fh <= G ? rot : v0));
    if (fh < G) sq[fh][fc] = v;
    else if (fh == G) skn[fc] = v;
    else svn[fc] = v;
  }
  __syncthreads();
  if (ls_w >= 0 && tid < 2 * HD) {
    const int pw = opaque(page_w);     // keeps the address arithmetic (and its wait) after the barrier
    T* dst = pool + (size_t)pw * a.page_elems;
    if (tid < HD) dst[((size_t)kvh * P + idx_w % P) * HD + tid] = from_f32<T>(skn[tid]);
    else dst[vofs + ((size_t)kvh * HD + (tid - HD)) * P + idx_w % P] = from_f32<T>(svn[tid - HD]);
  }

  const float sl2 = a.scale_log2;
  // The new key: p = exp2(0) = 1 against its own score; a partial result of its own.
  if (wave == 0 && ls_w >= 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      // lane c forms q[c] k[c], the wave sums them (a shuffle tree, not a 64-long chain)
      const float dot = wave_sum(lane_c ? sq[hh][lane] * skn[lane] : 0.f);
      if (lane == 0) { sm[NW][hh] = dot * sl2; sl[NW][hh] = 1.f; }
      if (lane_c) sacc[NW][hh][lane] = svn[lane];
    }
  }

  if constexpr (MF) {
    // query fragments (B operand of S^T): head fr (zero past G), head-dim elements 32 ks + 8 g ..+7
    bf16x8 qb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[ks][e] = (bf16)(fr < G ? sq[fr < G ? fr : 0][32 * ks + 8 * g + e] : 0.f);
    // this lane's head is fr (its scores, maximum and normaliser); its output rows are the heads
    // 4 g + e (only g = 0 holds heads, G <= 4), head-dim columns 16 hb + fr
    float m = -INFINITY, l = 0.f;
    f32x4 o[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) o[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool head_ok = fr < G;
    for (; t0 < nkeys; t0 += NW * KT) {
      f32x4 st[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][0], qb[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][1], qb[1], st[kb], 0, 0, 0);
      }
      // st[kb][e]: score of key t0 + 32 (kb / 2) + 8 g + 4 (kb % 2) + e for head fr
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = t0 + 32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + e;
          st[kb][e] = key < nkeys ? st[kb][e] * sl2 : -INFINITY;
          mx = fmaxf(mx, st[kb][e]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);                // the tile holds at least one key: finite
      const float alpha = exp2f(m - mn);            // 0 on the first tile (m = -inf)
      m = mn;
      l *= alpha;
      // rescale the output rows: head e's factor lives in lane e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ae = __shfl(alpha, e);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) o[hb][e] *= ae;
      }
      bf16x8 pf[2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = head_ok ? exp2f(st[kb][e] - mn) : 0.f;
          l += pv;
          pf[kb >> 1][4 * (kb & 1) + e] = (bf16)pv;
        }
      // the tile's V^T rows have landed in the wave's LDS tile (direct-to-LDS loads count as
      // vector memory loads)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // V^T fragments (B operand of P V: head-dim column 16 hb + fr, keys t0 + 32 ks + 8 g ..+7).
      // Keys past the context have zero probabilities; their page slots hold zeros or values an
      // earlier request stored (the pool is cleared at init), so every product term is finite.
      const char* vt = reinterpret_cast<const char*>(svt[wave]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 vv[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const int row = 16 * hb + fr;
          vv[hb] = *reinterpret_cast<const bf16x8*>(vt + row * 128 + (((4 * ks + g) ^ ((row >> 1) & 7)) << 4));
        }
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          o[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[ks], vv[hb], o[hb], 0, 0, 0);
      }
      if (t0 + NW * KT < nkeys) {
        // the next tile's V^T overwrites this one: every fragment read of it has completed
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        issue_tile(t0 + NW * KT, false);
      }
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (g == 0 && head_ok) { sm[wave][fr] = m; sl[wave][fr] = l; }
    if (g == 0) {
#pragma unroll
      for (int e = 0; e < G; ++e)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) sacc[wave][e][16 * hb + fr] = o[hb][e];
    }
  } else {
    float m[G], l[G], acc[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) { m[hh] = -INFINITY; l[hh] = 0.f; acc[hh] = 0.f; }
    for (; t0 < nkeys; t0 += NW * KT) {
      const int nt = min(KT, nkeys - t0);
      const bool valid = t0 + lane < nkeys;
      float sc[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) sc[hh] = 0.f;
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const float4 kv = kr32[c];
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
          sc[hh] += sq[hh][4 * c] * kv.x + sq[hh][4 * c + 1] * kv.y + sq[hh][4 * c + 2] * kv.z + sq[hh][4 * c + 3] * kv.w;
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float v = valid ? sc[hh] * sl2 : -INFINITY;
        float mt = v;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o));
        const float mn = fmaxf(m[hh], mt);
        const float alpha = exp2f(m[hh] - mn);
        const float p = valid ? exp2f(v - mn) : 0.f;
        l[hh] = l[hh] * alpha + wave_sum(p);
        acc[hh] *= alpha;
        m[hh] = mn;
        sp[wave][hh][lane] = p;
      }
      // this wave's probabilities are read back by the other lanes of the wave
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane_c) {
#pragma unroll
        for (int q = 0; q < KT / 4; ++q) {
          const float4 vv = vr32[q];
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            if (4 * q + 0 < nt) acc[hh] += sp[wave][hh][4 * q + 0] * vv.x;
            if (4 * q + 1 < nt) acc[hh] += sp[wave][hh][4 * q + 1] * vv.y;
            if (4 * q + 2 < nt) acc[hh] += sp[wave][hh][4 * q + 2] * vv.z;
            if (4 * q + 3 < nt) acc[hh] += sp[wave][hh][4 * q + 3] * vv.w;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (t0 + NW * KT < nkeys) issue_tile(t0 + NW * KT, false);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (lane == 0) { sm[wave][hh] = m[hh]; sl[wave][hh] = l[hh]; }
      if (lane_c) sacc[wave][hh][lane] = acc[hh];
    }
  }
  __syncthreads();
  // Wave hh merges query head hh: the waves that held keys in wave order, then the new key.
  const int nw_used = min(NW, (nkeys + KT - 1) / KT);
  if (wave < G && lane_c) {
    const int hh = wave;
    T* out = reinterpret_cast<T*>(a.o) + (size_t)s * a.nq;
    const bool with_new = ls_w >= 0;
    float M = -INFINITY;
    for (int w = 0; w < nw_used; ++w) M = fmaxf(M, sm[w][hh]);
    if (with_new) M = fmaxf(M, sm[NW][hh]);
    float L = 0.f, o = 0.f;
    for (int w = 0; w < nw_used; ++w) {
      const float f = exp2f(sm[w][hh] - M);
      L += sl[w][hh] * f;
      o += sacc[w][hh][lane] * f;
    }
    if (with_new) {
      const float f = exp2f(sm[NW][hh] - M);
      L += sl[NW][hh] * f;
      o += sacc[NW][hh][lane] * f;
    }
    out[(kvh * G + hh) * HD + lane] = from_f32<T>(o / L);
  }
}

template <typename T, int HD>
static hipError_t dec_attn_g(const DecArgs& a, int kind, int j, hipStream_t s) {
  dim3 grid(a.S, a.hkv);
  switch (a.hq / a.hkv) {
    case 1: hipLaunchKernelGGL((k_dec_attn<T, HD, 1>), grid, dim3(dec_attn_waves<T, HD, 1>() * 64), 0, s, a, kind, j); break;
    case 2: hipLaunchKernelGGL((k_dec_attn<T, HD, 2>), grid, dim3(dec_attn_waves<T, HD, 2>() * 64), 0, s, a, kind, j); break;
    case 3: hipLaunchKernelGGL((k_dec_attn<T, HD, 3>), grid, dim3(dec_attn_waves<T, HD, 3>() * 64), 0, s, a, kind, j); break;
    case 4: hipLaunchKernelGGL((k_dec_attn<T, HD, 4>), grid, dim3(dec_attn_waves<T, HD, 4>() * 64), 0, s, a, kind, j); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dec_attn(const DecArgs& a, int kind, int j, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {      // bf16 configurations have head dim 64
    return a.hd == 64 ? dec_attn_g<T, 64>(a, kind, j, s) : hipErrorInvalidValue;
  } else {
    switch (a.hd) {
      case 16: return dec_attn_g<T, 16>(a, kind, j, s);
      case 32: return dec_attn_g<T, 32>(a, kind, j, s);
      case 64: return dec_attn_g<T, 64>(a, kind, j, s);
      default: return hipErrorInvalidValue;
    }
  }
}
template hipError_t launch_dec_attn<float>(const DecArgs&, int, int, hipStream_t);
template hipError_t launch_dec_attn<bf16>(const DecArgs&, int, int, hipStream_t);

// ------------------------------------------------------------------ hand-over from a prefill
// Slot b takes request b, whose first T positions were computed by the prefill: its per-stream
// page lists are allocated in slot order from the free stack (one thread, in order), its
// recursion counts are the prefill's, and the next schedule admits its first decoded token at
// position T. Then every cached K/V row of the prefill is copied to its page (V transposed back).
__global__ void k_dec_prefix_alloc(DecArgs a, PrefixSrc p) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int top = a.glob[G_TOP];
  for (int b = 0; b < p.B; ++b) {
    a.sl_req[b] = b; a.sl_pos[b] = -1; a.sl_base[b] = p.T; a.sl_depth[b] = 0;
    for (int r = 0; r < a.R; ++r) a.sl_cnt[b * a.R + r] = p.cnt[r * p.cnt_ld + b];
    for (int ls = 0; ls < a.LS; ++ls) {
      int n;
      if (ls < 2) {
        n = p.T;
      } else {
        const int r = (ls - 2) / a.n_s + 1;
        n = (a.kv_share && r > 1) ? 0 : a.sl_cnt[b * a.R + r - 1];
      }
      const int np = (n + a.P - 1) / a.P;
      for (int i = 0; i < np; ++i) {
        if (top == 0) { a.glob[G_HALT] = 1; atomicOr(a.err, (unsigned)ERR_KV_FULL); a.glob[G_TOP] = 0; return; }
        a.ptab[((size_t)b * a.LS + ls) * a.pps + i] = a.free_pages[--top];
      }
    }
  }
  a.glob[G_TOP] = top;
  a.glob[G_NEXT] = p.B;
  a.glob[G_PEAK] = a.kv_pages - top;
}

// One thread per (sequence, prefill stream, cached row, element of K or V).
template <typename T>
__global__ void k_dec_prefix_copy(DecArgs a, PrefixSrc p, int nstreams) {
  const int HDk = a.hd, row = a.hkv * HDk;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long per_seq = (long long)nstreams * p.T * 2 * row;
  if (i >= per_seq * p.B || a.glob[G_HALT]) return;
  const int b = (int)(i / per_seq);
  long long rem = i - b * per_seq;
  const int ps = (int)(rem / ((long long)p.T * 2 * row));
  rem -= (long long)ps * p.T * 2 * row;
  const int idx = (int)(rem / (2 * row));
  const int e = (int)(rem - (long long)idx * 2 * row);
  const bool isv = e >= row;
  const int h = (e % row) / HDk, c = e % HDk;
  // prefill stream -> layer stream and number of cached rows
  const int last = nstreams - 1;
  int ls, n;
  if (ps == 0) { ls = 0; n = p.T; }
  else if (ps == last) { ls = 1; n = p.T; }
  else {
    const int r = (ps - 1) / a.n_s + 1;
    ls = ps + 1;
    n = (a.kv_share && r > 1) ? 0 : p.cnt[(r - 1) * p.cnt_ld + b];
  }
  if (idx >= n) return;
  const T* k = reinterpret_cast<const T*>(reinterpret_cast<const char*>(p.kv) + (size_t)ps * 2 * p.half_bytes);
  const T* vt = reinterpret_cast<const T*>(reinterpret_cast<const char*>(p.kv) + ((size_t)ps * 2 + 1) * p.half_bytes);
  const T v = isv ? vt[(((size_t)b * a.hkv + h) * HDk + c) * p.kpad + idx]
                  : k[((size_t)b * p.kpad + idx) * row + h * HDk + c];
  const int page = a.ptab[((size_t)b * a.LS + ls) * a.pps + idx / a.P];
  T* dst = reinterpret_cast<T*>(a.pool) + (size_t)page * a.page_elems +
           (isv ? (size_t)a.hkv * a.P * HDk + ((size_t)h * HDk + c) * a.P + idx % a.P
                : ((size_t)h * a.P + idx % a.P) * HDk + c);
  *dst = v;
}

hipError_t launch_dec_prefix(const DecArgs& a, const PrefixSrc& p, hipStream_t s) {
  hipLaunchKernelGGL(k_dec_prefix_alloc, dim3(1), dim3(64), 0, s, a, p);
  const int nstreams = 2 + a.R * a.n_s;
  const long long total = (long long)p.B * nstreams * p.T * 2 * a.hkv * a.hd;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (a.es == 2) hipLaunchKernelGGL((k_dec_prefix_copy<bf16>), dim3(blocks), dim3(256), 0, s, a, p, nstreams);
  else hipLaunchKernelGGL((k_dec_prefix_copy<float>), dim3(blocks), dim3(256), 0, s, a, p, nstreams);
  return hipGetLastError();
}

// ------------------------------------------------------------------ skinny projections
// out^T = W . A^T for the 64 rows of A (the slots), weights on the MFMA A side. A workgroup owns
// RG groups of 16 weight rows and one contiguous range of 128-byte K slices (K is split over
// grid.y so that enough CUs stream the weights); its 4 waves take the range's slices in turn,
// loading the fragments of SK_BATCH of their slices before multiplying them (SK_BATCH is the
// number of slices a wave has, up to 4, so one round of loads usually covers them; several loads per
// lane in flight), and add their partial sums in wave order in LDS (deterministic). Wave w then
// finishes slot rows 16w..16w+15: each lane holds 4 consecutive output columns of one row.
constexpr int SK_WAVES = 4;

template <typename T, int RG, int EPI, int SK_BATCH>
__global__ __launch_bounds__(SK_WAVES * 64) void k_skinny(const T* __restrict__ A,
                                                          const T* __restrict__ W, int N, int K,
                                                          int M, SkinnyEpi ep) {
  typedef Mma<T> MM;
  constexpr int UK = 128 / (int)sizeof(T);          // K elements per slice
  constexpr int NS = UK / MM::KSTEP;               // MFMA steps per slice
  __shared__ f32x4 red[SK_WAVES][RG][4][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16 * RG;
  const int nu = K / UK;
  const int per = (nu + gridDim.y - 1) / gridDim.y;
  const int ulo = blockIdx.y * per, uhi = min(nu, ulo + per);
  f32x4 acc[RG][4];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int mf = 0; mf < 4; ++mf) acc[rg][mf] = f32x4{0.f, 0.f, 0.f, 0.f};

  const T* wrow[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) wrow[rg] = W + (size_t)(n0 + 16 * rg + fr) * K + g * MM::KW;
  // slot rows at or past M are not loaded (their fragments stay zero and their outputs unused):
  // with 51 of 64 rows in use that is a fifth less activation traffic per workgroup
  const T* arow[4];
  bool arow_in[4];
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
    arow[mf] = A + (size_t)(16 * mf + fr) * K + g * MM::KW;
    arow_in[mf] = 16 * mf + fr < M;
  }

  for (int u0 = ulo + wave; u0 < uhi; u0 += SK_WAVES * SK_BATCH) {
    typename MM::frag wa[SK_BATCH][RG][NS], xb[SK_BATCH][4][NS];
#pragma unroll
    for (int bt = 0; bt < SK_BATCH; ++bt) {
      const int u = min(u0 + bt * SK_WAVES, uhi - 1);  // past the range: a repeated slice, zeroed below
#pragma unroll
      for (int ks = 0; ks < NS; ++ks) {
        const int k = u * UK + ks * MM::KSTEP;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) wa[bt][rg][ks] = MM::load(wrow[rg] + k);
#pragma unroll
        for (int mf = 0; mf < 4; ++mf)
          xb[bt][mf][ks] = arow_in[mf] ? MM::load(arow[mf] + k) : typename MM::frag{};
      }
    }
    // keep every load of the batch ahead of the multiplies (several loads in flight per lane)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int bt = 0; bt < SK_BATCH; ++bt) {
      if (u0 + bt * SK_WAVES >= uhi) {             // repeated slice: multiply zeros instead
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int ks = 0; ks < NS; ++ks) wa[bt][rg][ks] = typename MM::frag{};
      }
#pragma unroll
      for (int ks = 0; ks < NS; ++ks)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int mf = 0; mf < 4; ++mf) acc[rg][mf] = MM::mma(wa[bt][rg][ks], xb[bt][mf][ks], acc[rg][mf]);
    }
  }
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int mf = 0; mf < 4; ++mf) red[wave][rg][mf][lane] = acc[rg][mf];
  __syncthreads();
  const int mf = wave;
  f32x4 v[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    v[rg] = red[0][rg][mf][lane];
#pragma unroll
    for (int w = 1; w < SK_WAVES; ++w) v[rg] += red[w][rg][mf][lane];
  }
  const int m = 16 * mf + fr;
  if (m >= M) return;
  if constexpr (EPI == SK_PARTIAL) {
    float* out = ep.out + (size_t)blockIdx.y * 64 * ep.ldo;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const int n = n0 + 16 * rg + 4 * g;
      *reinterpret_cast<float4*>(out + (size_t)m * ep.ldo + n) =
          make_float4(v[rg][0], v[rg][1], v[rg][2], v[rg][3]);
    }
  } else {  // SK_SWIGLU: weight rows are gate/up groups of 16 (RG == 2)
    const int col = (n0 >> 1) + 4 * g;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gt = v[0][e], up = v[1][e];
      o[e] = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
    }
    Vec4<T>::store(reinterpret_cast<T*>(ep.h) + (size_t)m * ep.ldh + col, o[0], o[1], o[2], o[3]);
  }
}

template <typename T>
hipError_t launch_skinny(int epi, const T* A, const T* W, int N, int K, int M, int ksplit,
                         const SkinnyEpi& ep, hipStream_t s) {
  if (K % 64 || N % 32 || M > 64 || ksplit < 1 || ksplit > 8) return hipErrorInvalidValue;
  // slices each wave handles: the batch covers them in one round of loads where registers allow
  const int uk = 128 / (int)sizeof(T), per_split = (K / uk + ksplit - 1) / ksplit;
  const int per_wave = (per_split + SK_WAVES - 1) / SK_WAVES;
  const dim3 blk(SK_WAVES * 64);
  if (epi == SK_PARTIAL) {
    const dim3 grid(N / 16, ksplit);
    if (per_wave <= 1) hipLaunchKernelGGL((k_skinny<T, 1, SK_PARTIAL, 1>), grid, blk, 0, s, A, W, N, K, M, ep);
    else if (per_wave == 2) hipLaunchKernelGGL((k_skinny<T, 1, SK_PARTIAL, 2>), grid, blk, 0, s, A, W, N, K, M, ep);
    else if (per_wave == 3) hipLaunchKernelGGL((k_skinny<T, 1, SK_PARTIAL, 3>), grid, blk, 0, s, A, W, N, K, M, ep);
    else hipLaunchKernelGGL((k_skinny<T, 1, SK_PARTIAL, 4>), grid, blk, 0, s, A, W, N, K, M, ep);
  } else {
    if (ksplit != 1) return hipErrorInvalidValue;
    const dim3 grid(N / 32, 1);
    if (per_wave <= 1) hipLaunchKernelGGL((k_skinny<T, 2, SK_SWIGLU, 1>), grid, blk, 0, s, A, W, N, K, M, ep);
    else if (per_wave == 2) hipLaunchKernelGGL((k_skinny<T, 2, SK_SWIGLU, 2>), grid, blk, 0, s, A, W, N, K, M, ep);
    else if (per_wave == 3) hipLaunchKernelGGL((k_skinny<T, 2, SK_SWIGLU, 3>), grid, blk, 0, s, A, W, N, K, M, ep);
    else hipLaunchKernelGGL((k_skinny<T, 2, SK_SWIGLU, 4>), grid, blk, 0, s, A, W, N, K, M, ep);
  }
  return hipGetLastError();
}
template hipError_t launch_skinny<float>(int, const float*, const float*, int, int, int, int, const SkinnyEpi&, hipStream_t);
template hipError_t launch_skinny<bf16>(int, const bf16*, const bf16*, int, int, int, int, const SkinnyEpi&, hipStream_t);

}  // namespace mor
