// Capacity-bounded permutation of the MoE layer (gfx950): expert histogram,
// exclusive scan, capacity, stable token-order slots, drop mask, and the row
// scatter into fixed-capacity per-expert buckets.
//
// Sources: "Expert Parallelism" (inferensys.com glossary), capacity entry
// (an expert takes at most C = cf*k*T/E tokens; the excess is dropped) and
// memory entry (pre-allocated contiguous buffers of maximum capacity);
// "Expert Parallelism & All-to-All" (neelmishra.github.io), "Why fixed-size
// buffers matter here" (fixed per-expert buffer; drops on overflow, padding on
// underflow) and "Why MoE forces a new axis" (E/P whole experts per device).
//
// Slot of copy i = t*k + j of expert e: the number of earlier copies (in
// flattened token order) of the same expert. It is found as
//   tile offset (scan of per-tile counts over earlier tiles)
// + rank inside the tile (wave ballots over the expert-id bits).
// Positions never come from atomics; only the order-free per-tile counts do.
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

// Per-tile expert histogram: tile_cnt[b][e] = copies of expert e among tokens
// [64 b, 64 b + 64). Entries outside [0, E) are counted nowhere (dropped).
__global__ __launch_bounds__(256) void tile_hist_kernel(const int32_t* __restrict__ idx,
                                                        int64_t T, int k, int E,
                                                        int32_t* __restrict__ tile_cnt) {
  extern __shared__ int hist[];
  const int64_t b = blockIdx.x;
  const int64_t t0 = b * kTileTokens;
  const int n = static_cast<int>(min<int64_t>(kTileTokens, T - t0)) * k;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = idx[t0 * k + i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) tile_cnt[b * E + e] = hist[e];
}

// Exclusive scan of one int per thread over a block of 1024 threads.
__device__ int block_exclusive_scan_1024(int v, int* total, int* sh /* >= 17 ints */) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = sh[w];
      sh[w] = run;
      run += t;
    }
    sh[16] = run;
  }
  __syncthreads();
  const int out = sh[wave] + incl - v;
  *total = sh[16];
  __syncthreads();
  return out;
}

// mtile_off[e] = sum over e' < e of ceil(kept[e'] / bm); mtile_off[E] = total.
// Block of 1024 threads, 4 experts per thread (E <= 4096).
__device__ void mtile_prefix(const int* kept_s, int E, int bm, int32_t* mtile_off, int* sh) {
  int v[4];
  int local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    v[q] = e < E ? (kept_s[e] + bm - 1) / bm : 0;
    local += v[q];
  }
  int total;
  int run = block_exclusive_scan_1024(local, &total, sh);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    if (e < E) mtile_off[e] = run;
    run += v[q];
  }
  if (threadIdx.x == 0) mtile_off[E] = total;
}

// Exclusive scan over tiles per expert, then counts, totals, send counts and
// the GEMM row-tile map; one block of 1024 threads. The scan takes 64 experts
// at a time with 16 lanes each; lane ly owns a contiguous run of tiles.
__global__ __launch_bounds__(1024) void scan_finalize_kernel(
    const int32_t* __restrict__ tile_cnt, int64_t nt, int E, int64_t C, int P, int64_t row_bytes, int k,
    int64_t T, int32_t* __restrict__ tile_off, int32_t* __restrict__ routed, int32_t* __restrict__ kept,
    int32_t* __restrict__ send, int64_t* __restrict__ totals, int bm, int32_t* __restrict__ mtile_off,
    const int32_t* __restrict__ place) {
  __shared__ int part[16][65];
  __shared__ int kept_s[4096];
  __shared__ int send_s[4096];  // kept rows per rank (P <= E)
  __shared__ int sh[17];
  __shared__ unsigned long long ksum;
  const int ex = threadIdx.x & 63;
  const int ly = threadIdx.x >> 6;
  const int64_t chunk = ceil_div(nt, 16);
  const int64_t b0 = min(nt, ly * chunk);
  const int64_t b1 = min(nt, b0 + chunk);
  const int per = E / P;
  if (threadIdx.x == 0) ksum = 0;
  for (int p = threadIdx.x; p < P; p += blockDim.x) send_s[p] = 0;  // ordered by the first barrier below
  for (int eb = 0; eb < E; eb += 64) {
    const int e = eb + ex;
    int sum = 0;
    if (e < E)
      for (int64_t b = b0; b < b1; ++b) sum += tile_cnt[b * E + e];
    part[ly][ex] = sum;
    __syncthreads();
    int run = 0;
    for (int l = 0; l < ly; ++l) run += part[l][ex];
    if (e < E) {
      for (int64_t b = b0; b < b1; ++b) {
        const int v = tile_cnt[b * E + e];
        tile_off[b * E + e] = run;
        run += v;
      }
      if (ly == 15) {
        routed[e] = run;
        const int kv = static_cast<int>(min<int64_t>(run, C));
        kept[e] = kv;
        kept_s[e] = kv;
        atomicAdd(&ksum, static_cast<unsigned long long>(kv));  // integer sums: order-free
        atomicAdd(&send_s[place ? place[e] : e / per], kv);
      }
    }
    __syncthreads();
  }
  if (send)
    for (int p = threadIdx.x; p < P; p += blockDim.x) send[p] = send_s[p];
  if (totals && threadIdx.x == 0) {
    const int64_t n_kept = static_cast<int64_t>(ksum);
    const int64_t rank0 = send_s[0];
    totals[0] = T * k - n_kept;
    totals[1] = 0;  // fully dropped tokens: accumulated by the slot kernel
    totals[2] = static_cast<int64_t>(E) * C - n_kept;
    totals[3] = (n_kept - rank0) * row_bytes;
  }
  if (mtile_off) mtile_prefix(kept_s, E, bm, mtile_off, sh);
}

// Row-tile map from counts given by the caller: each count is clamped to
// [0, C] first, so no tile starts past an expert's bucket.
__global__ __launch_bounds__(1024) void mtile_map_kernel(const int32_t* __restrict__ kept, int E, int64_t C,
                                                         int bm, int32_t* __restrict__ mtile_off) {
  __shared__ int kept_s[4096];
  __shared__ int sh[17];
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    kept_s[e] = static_cast<int>(min(max(static_cast<int64_t>(kept[e]), int64_t{0}), C));
  __syncthreads();
  mtile_prefix(kept_s, E, bm, mtile_off, sh);
}

// src[e][s] = -1 on padding rows s >= kept[e] (kept rows come from the slot kernel).
__global__ __launch_bounds__(256) void src_padding_kernel(const int32_t* __restrict__ kept,
                                                          int64_t C, int E,
                                                          int32_t* __restrict__ src) {
  const int e = blockIdx.y;
  for (int64_t s = kept[e] + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; s < C;
       s += static_cast<int64_t>(gridDim.x) * blockDim.x)
    src[e * C + s] = -1;
}

// Slots of one 64-token tile, one wave. Copies are taken 64 at a time in
// flattened order; lanes with the same expert form a group found by ballots
// over the expert-id bits; a lane's rank is the number of group lanes below
// it. The group's highest lane advances the expert's running count.
// With route_off (the exclusive scan of the routed counts), every routed copy,
// kept or dropped, is also listed per expert in token order: entry
// route_off[e] + rank holds the copy's flat index (lcopy) and token (ltok).
__global__ __launch_bounds__(64) void slots_kernel(const int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ tile_off,
                                                   int64_t T, int k, int E, int64_t C,
                                                   int32_t* __restrict__ slot,
                                                   int32_t* __restrict__ src,
                                                   int64_t* __restrict__ totals,
                                                   const int32_t* __restrict__ route_off,
                                                   int32_t* __restrict__ lcopy,
                                                   int32_t* __restrict__ ltok) {
  extern __shared__ int sm[];
  int* cnt = sm;          // [E]
  int* sbuf = sm + E;     // [64 * k]
  const int lane = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t t0 = b * kTileTokens;
  const int n = static_cast<int>(min<int64_t>(kTileTokens, T - t0));
  const int ncp = n * k;
  for (int e = lane; e < E; e += 64) cnt[e] = tile_off[b * E + e];
  __syncthreads();
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  // every copy of the tile up front: at most 64 * 32 / 64 = 32 per lane
  int ev[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const int i = c * 64 + lane;
    ev[c] = i < ncp ? idx[t0 * k + i] : 0;
  }
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const int base = c * 64;
    if (base >= ncp) break;
    const int i = base + lane;
    const bool valid = static_cast<unsigned>(ev[c]) < static_cast<unsigned>(E);  // else dropped
    const bool active = i < ncp && valid;
    const int e = valid ? ev[c] : 0;
    unsigned long long mask = __ballot(active);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (e >> bit) & 1;
      const unsigned long long m = __ballot(active && set);
      mask &= set ? m : ~m;
    }
    const int rank = __popcll(mask & below);
    const int s = active ? cnt[e] + rank : 0;
    __syncthreads();
    if (active && (63 - __clzll(mask)) == lane) cnt[e] = s + 1;
    __syncthreads();
    if (i < ncp && !valid) {
      slot[t0 * k + i] = -1;
      sbuf[i] = -1;
    }
    if (active) {
      const int sl = s < C ? s : -1;
      slot[t0 * k + i] = sl;
      sbuf[i] = sl;
      if (src && sl >= 0) src[static_cast<int64_t>(e) * C + s] = static_cast<int32_t>(t0 * k + i);
      if (route_off) {
        const int64_t at = static_cast<int64_t>(route_off[e]) + s;
        lcopy[at] = static_cast<int32_t>(t0 * k + i);
        ltok[at] = static_cast<int32_t>(t0 + i / k);
      }
    }
  }
  __syncthreads();
  if (totals) {
    bool all_dropped = lane < n;
    for (int j = 0; j < k && all_dropped; ++j) all_dropped = sbuf[lane * k + j] < 0;
    const int c = __popcll(__ballot(all_dropped));
    if (lane == 0 && c) atomicAdd(reinterpret_cast<unsigned long long*>(&totals[1]),
                                  static_cast<unsigned long long>(c));
  }
}

// Row scatter: one 256-thread block per token moves its row (16-byte words,
// U per lane, so a row of up to 256*U words takes one pass) to each kept
// destination bucket row; the row is read once and written k' <= k times with
// streaming stores. Lane j of each wave loads copy j's slot and expert (k <=
// 32) while the row's words are on their way, and a ballot over the slots
// gives the kept copies.
template <int U>
__global__ __launch_bounds__(256) void scatter_rows_kernel(const uint4* __restrict__ x,
                                                           const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ slot, int64_t T,
                                                           int k, int64_t C, int64_t V,
                                                           uint4* __restrict__ buckets) {
  const int64_t t = blockIdx.x;
  if (t >= T) return;
  const int lane = threadIdx.x;
  const int wl = threadIdx.x % 64;
  int s_l = -1, e_l = 0;
  if (wl < k) {
    s_l = slot[t * k + wl];
    e_l = idx[t * k + wl];
  }
  const uint4* xr = x + t * V;
  // taken while every lane is active: lanes past the row's end leave the loop below
  const uint64_t kept = __ballot(s_l >= 0);
  for (int64_t v0 = lane; v0 < V; v0 += 256 * U) {
    uint4 val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + 256 * u;
      if (v < V) val[u] = xr[v];
    }
    for (uint64_t m = kept; m; m &= m - 1) {
      const int j = __builtin_ctzll(m);
      const int e = __builtin_amdgcn_readlane(e_l, j);
      const int sl = __builtin_amdgcn_readlane(s_l, j);
      uint4* dst = buckets + (static_cast<int64_t>(e) * C + sl) * V;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + 256 * u;
        if (v < V) store_stream(&dst[v], val[u]);
      }
    }
  }
}

// Replica layout, one block: inst_off [E+1] = exclusive prefix of the replica
// counts (each taken as at least 1), expert of each instance (wmap [R]) and its
// rank (place [R]): replica j of expert e on rank (e / (E/P) + j) mod P.
__global__ __launch_bounds__(1024) void replica_layout_kernel(const int32_t* __restrict__ replicas, int E, int R,
                                                              int P, int32_t* __restrict__ inst_off,
                                                              int32_t* __restrict__ wmap,
                                                              int32_t* __restrict__ place) {
  __shared__ int sh[17];
  for (int i = threadIdx.x; i < R; i += blockDim.x) {  // instances no replica reaches: expert 0, rank 0
    wmap[i] = 0;
    place[i] = 0;
  }
  int v[4];
  int local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    v[q] = e < E ? max(replicas[e], 1) : 0;
    local += v[q];
  }
  int total;
  int run = block_exclusive_scan_1024(local, &total, sh);
  const int per = E / P;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    if (e >= E) continue;
    inst_off[e] = run;
    for (int j = 0; j < v[q] && run + j < R; ++j) {
      wmap[run + j] = e;
      place[run + j] = (e / per + j) % P;
    }
    run += v[q];
  }
  if (threadIdx.x == 0) inst_off[E] = total;
}

// Instance of each copy: copy (t, j) of expert e with token-order rank q among
// e's copies goes to instance inst_off[e] + q mod r (clamped below R).
__global__ __launch_bounds__(256) void instance_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ qrank,
                                                       const int32_t* __restrict__ replicas,
                                                       const int32_t* __restrict__ inst_off, int64_t n, int R,
                                                       int32_t* __restrict__ inst) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int e = idx[i];
    const int r = max(replicas[e], 1);
    inst[i] = min(inst_off[e] + qrank[i] % r, R - 1);
  }
}

}  // namespace

hipError_t launch_tile_hist(const int32_t* idx, int64_t T, int k, int E, int32_t* tile_cnt,
                            hipStream_t s) {
  const int64_t nt = ceil_div(T, kTileTokens);
  if (nt == 0) return hipSuccess;
  tile_hist_kernel<<<dim3(static_cast<unsigned>(nt)), dim3(256), E * sizeof(int), s>>>(idx, T, k, E,
                                                                                     tile_cnt);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* tile_cnt, int64_t nt, int E, int64_t C, int P,
                       int64_t row_bytes, int k, int64_t T, int32_t* tile_off, int32_t* routed,
                       int32_t* kept, int32_t* send, int64_t* totals, int bm, int32_t* mtile_off,
                       int32_t* src, hipStream_t s, const int32_t* place) {
  scan_finalize_kernel<<<dim3(1), dim3(1024), 0, s>>>(tile_cnt, nt, E, C, P, row_bytes, k, T, tile_off, routed,
                                                      kept, send, totals, bm, mtile_off, place);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !src) return err;
  const unsigned gx = static_cast<unsigned>(std::min<int64_t>(ceil_div(C, 256), 64));
  src_padding_kernel<<<dim3(gx, static_cast<unsigned>(E)), dim3(256), 0, s>>>(kept, C, E, src);
  return hipGetLastError();
}

hipError_t launch_mtile_map(const int32_t* kept, int E, int64_t C, int bm, int32_t* mtile_off, hipStream_t s) {
  mtile_map_kernel<<<dim3(1), dim3(1024), 0, s>>>(kept, E, C, bm, mtile_off);
  return hipGetLastError();
}

hipError_t launch_slots(const int32_t* idx, const int32_t* tile_off, int64_t T, int k, int E,
                        int64_t C, int32_t* slot, int32_t* src, int64_t* totals, hipStream_t s,
                        const int32_t* route_off, int32_t* lcopy, int32_t* ltok) {
  const int64_t nt = ceil_div(T, kTileTokens);
  if (nt == 0) return hipSuccess;
  if (route_off && (!lcopy || !ltok)) return hipErrorInvalidValue;
  const size_t shm = (static_cast<size_t>(E) + static_cast<size_t>(kTileTokens) * k) * sizeof(int);
  slots_kernel<<<dim3(static_cast<unsigned>(nt)), dim3(64), shm, s>>>(idx, tile_off, T, k, E, C,
                                                                     slot, src, totals, route_off, lcopy, ltok);
  return hipGetLastError();
}

namespace {
// Exclusive scan of n int32 counts by one block: thread t sums a contiguous
// run, the run totals are scanned in LDS, then each run is written out.
__global__ __launch_bounds__(1024) void exclusive_scan_kernel(const int32_t* __restrict__ in, int n,
                                                              int32_t* __restrict__ out) {
  __shared__ int32_t tot[1024];
  const int t = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int a = min(n, t * per), b = min(n, a + per);
  int32_t sum = 0;
  for (int i = a; i < b; ++i) sum += in[i];
  tot[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int32_t v = t >= off ? tot[t - off] : 0;
    __syncthreads();
    tot[t] += v;
    __syncthreads();
  }
  int32_t run = tot[t] - sum;
  for (int i = a; i < b; ++i) {
    out[i] = run;
    run += in[i];
  }
  if (t == 1023) out[n] = tot[1023];
}
}  // namespace

hipError_t launch_exclusive_scan(const int32_t* in, int n, int32_t* out, hipStream_t s) {
  if (n < 0) return hipErrorInvalidValue;
  exclusive_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(in, n, out);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const void* x, const int32_t* idx, const int32_t* slot, int64_t T,
                               int k, int64_t C, int64_t row_bytes, void* buckets, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const auto* xv = static_cast<const uint4*>(x);
  auto* bv = static_cast<uint4*>(buckets);
  if (k > 32) return hipErrorInvalidValue;  // one lane per copy, k <= 32 lanes of a wave
  const int64_t V = row_bytes / 16;
  const dim3 grid(static_cast<unsigned>(T));
  // words per lane: the smallest of 1, 2, 4 that covers the row in one pass, else 8
  if (V <= 256)
    scatter_rows_kernel<1><<<grid, dim3(256), 0, s>>>(xv, idx, slot, T, k, C, V, bv);
  else if (V <= 512)
    scatter_rows_kernel<2><<<grid, dim3(256), 0, s>>>(xv, idx, slot, T, k, C, V, bv);
  else if (V <= 1024)
    scatter_rows_kernel<4><<<grid, dim3(256), 0, s>>>(xv, idx, slot, T, k, C, V, bv);
  else
    scatter_rows_kernel<8><<<grid, dim3(256), 0, s>>>(xv, idx, slot, T, k, C, V, bv);
  return hipGetLastError();
}

hipError_t launch_replica_layout(const int32_t* replicas, int E, int R, int P, int32_t* inst_off, int32_t* wmap,
                                 int32_t* place, hipStream_t s) {
  replica_layout_kernel<<<dim3(1), dim3(1024), 0, s>>>(replicas, E, R, P, inst_off, wmap, place);
  return hipGetLastError();
}

hipError_t launch_instances(const int32_t* idx, const int32_t* qrank, const int32_t* replicas,
                            const int32_t* inst_off, int64_t n, int R, int32_t* inst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  instance_kernel<<<dim3(static_cast<unsigned>(std::min<int64_t>(ceil_div(n, 256), 4096))), dim3(256), 0, s>>>(
      idx, qrank, replicas, inst_off, n, R, inst);
  return hipGetLastError();
}

}  // namespace moe
