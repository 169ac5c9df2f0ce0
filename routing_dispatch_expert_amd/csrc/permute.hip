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
// + rank inside the tile (wave ballots over the expert-id bits; computed with
//   the tile histogram, by the route kernel or tile_hist_kernel).
// Positions never come from atomics; the only atomics are order-free integer
// sums (per-rank send counts over a replica placement, fully dropped tokens).
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

// Per-tile expert histogram and ranks: tile_cnt[b][e] = copies of expert e
// among tokens [64 b, 64 b + 64), and rank [T, k] (optional) of each copy
// within its tile; *zero = 0 when given. Entries outside [0, E) are counted nowhere and ranked -1
// (dropped). One 1024-thread block per tile; all 16 waves rank the tile's
// copies (rank_tile_waves) when its chunk counts fit LDS (k <= 16, k E <=
// 8192), else one wave (rank_tile).
__global__ __launch_bounds__(1024) void tile_hist_kernel(const int32_t* __restrict__ idx,
                                                         int64_t T, int k, int E,
                                                         int32_t* __restrict__ tile_cnt,
                                                         int32_t* __restrict__ rank, int64_t* zero) {
  extern __shared__ int sm[];
  if (zero && blockIdx.x == 0 && threadIdx.x == 0) *zero = 0;
  int* hist = sm;                        // [E]
  int* ecp = sm + E;                     // [64 k]
  int* cc = ecp + kTileTokens * k;       // [k E] for the all-wave ranking
  const int64_t b = blockIdx.x;
  const int64_t t0 = b * kTileTokens;
  const int n = static_cast<int>(min<int64_t>(kTileTokens, T - t0)) * k;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = idx[t0 * k + i];
    ecp[i] = static_cast<unsigned>(e) < static_cast<unsigned>(E) ? e : -1;
  }
  lds_barrier();
  int32_t* rk = rank ? rank + t0 * k : nullptr;
  if (tile_ranks_by_waves(k, E)) {
    rank_tile_waves(ecp, n, E, hist, cc, rk);
  } else {
    if (threadIdx.x < 64) rank_tile(ecp, n, E, hist, rk);
    lds_barrier();
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) tile_cnt[b * E + e] = hist[e];
}

// Exclusive scan of one int per thread over a block of 1024 threads. Its
// barriers order LDS only: global stores issued before it may still be in
// flight after it.
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
  lds_barrier();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = sh[w];
      sh[w] = run;
      run += t;
    }
    sh[16] = run;
  }
  lds_barrier();
  const int out = sh[wave] + incl - v;
  *total = sh[16];
  lds_barrier();
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

// Per-rank send counts, totals and the GEMM row-tile maps from the kept
// counts in LDS (one block of 1024 threads). kpre [E + 1] and send_s [P] are
// LDS scratch. The send counts are differences of the kept prefix (rank p
// holds experts [p E/P, (p+1) E/P)), or LDS sums over `place` when given.
struct ScanTail {
  int64_t C, row_bytes, T;
  int E, P, k;
  int32_t* send;
  int64_t* totals;
  int bm0, bm1;
  int32_t *mtile0, *mtile1;
  const int32_t* place;
  int32_t* clear;  // zeroed when given: n_clear words
  int n_clear;
  bool leave_t1;   // totals[1] is zeroed before the scan and counted beside it
};

__device__ void scan_tail(const ScanTail& a, const int* kept_s, int* kpre, int* send_s, int* sh) {
  const int tid = threadIdx.x;
  int v[4];
  int local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    v[q] = e < a.E ? kept_s[e] : 0;
    local += v[q];
  }
  int n_kept;  // at most T k copies: fits an int like the copy indices
  int run = block_exclusive_scan_1024(local, &n_kept, sh);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < a.E) kpre[e] = run;
    run += v[q];
  }
  if (tid == 0) kpre[a.E] = n_kept;
  if (a.place)
    for (int p = tid; p < a.P; p += blockDim.x) send_s[p] = 0;
  lds_barrier();
  const int per = a.E / a.P;
  if (a.place) {
    for (int e = tid; e < a.E; e += blockDim.x) atomicAdd(&send_s[a.place[e]], kept_s[e]);  // order-free
    lds_barrier();
  }
  if (a.send)
    for (int p = tid; p < a.P; p += blockDim.x)
      a.send[p] = a.place ? send_s[p] : kpre[(p + 1) * per] - kpre[p * per];
  if (a.totals && tid == 0) {
    const int send0 = a.place ? send_s[0] : kpre[per];
    a.totals[0] = a.T * a.k - n_kept;
    if (!a.leave_t1) a.totals[1] = 0;  // fully dropped tokens: added by the slot kernel that follows
    a.totals[2] = static_cast<int64_t>(a.E) * a.C - n_kept;
    a.totals[3] = static_cast<int64_t>(n_kept - send0) * a.row_bytes;
  }
  if (a.mtile0) mtile_prefix(kept_s, a.E, a.bm0, a.mtile0, sh);
  if (a.mtile1) mtile_prefix(kept_s, a.E, a.bm1, a.mtile1, sh);
  if (a.clear)
    for (int i = tid; i < a.n_clear; i += blockDim.x) a.clear[i] = 0;
}

// The scan, one block of 1024 threads: per expert, the exclusive prefix over
// tiles of its tile counts (tile_off), then the routed and kept counts and
// the tail. Experts are taken EB at a time (EB = 64 .. 1024, a power of two
// covering E where it can), 1024 / EB lanes per expert; lane ly sums a
// contiguous run of tiles, the runs are scanned in LDS, and each lane writes
// its run's offsets. The first F counts of a run are loaded at once and stay
// in registers between the two passes; the rest go out eight at a time.
template <int F>
__device__ void scan_block(const int32_t* __restrict__ tile_cnt, int64_t nt, int32_t* __restrict__ tile_off,
                           int32_t* __restrict__ routed, int32_t* __restrict__ kept, const ScanTail& tail,
                           int* sm /* dynamic LDS: 2 E + 1 + P ints */) {
  const int E = tail.E;
  int* kept_s = sm;              // [E]
  int* kpre = sm + E;            // [E + 1]
  int* send_s = kpre + E + 1;    // [P]
  __shared__ int part[1024];
  __shared__ int sh[17];
  const int EB = E <= 64 ? 64 : (E <= 128 ? 128 : (E <= 256 ? 256 : (E <= 512 ? 512 : 1024)));
  const int LY = 1024 / EB;
  const int tid = threadIdx.x, ex = tid % EB, ly = tid / EB;
  const int ntt = static_cast<int>(nt);  // nt E < 2^31 (checked by the launcher)
  const int chunk = (ntt + LY - 1) / LY;
  const int b0 = min(ntt, ly * chunk);
  const int b1 = min(ntt, b0 + chunk);
  constexpr int B = 8;  // loads per batch
  for (int base = 0; base < E; base += EB) {
    const int e = base + ex;
    int first[F];
    int sum = 0;
    if (e < E) {
#pragma unroll
      for (int j = 0; j < F; ++j) {
        first[j] = b0 + j < b1 ? tile_cnt[(b0 + j) * E + e] : 0;
        sum += first[j];
      }
      for (int b = b0 + F; b < b1; b += B) {
        int v[B];
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] = b + j < b1 ? tile_cnt[(b + j) * E + e] : 0;
#pragma unroll
        for (int j = 0; j < B; ++j) sum += v[j];
      }
    }
    part[tid] = sum;
    lds_barrier();
    int run = 0;
    for (int l = 0; l < ly; ++l) run += part[l * EB + ex];
    if (e < E) {
#pragma unroll
      for (int j = 0; j < F; ++j)
        if (b0 + j < b1) {
          tile_off[(b0 + j) * E + e] = run;
          run += first[j];
        }
      for (int b = b0 + F; b < b1; b += B) {
        int v[B];
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] = b + j < b1 ? tile_cnt[(b + j) * E + e] : 0;
#pragma unroll
        for (int j = 0; j < B; ++j)
          if (b + j < b1) {
            tile_off[(b + j) * E + e] = run;
            run += v[j];
          }
      }
      if (ly == LY - 1) {
        const int kv = static_cast<int>(min<int64_t>(run, tail.C));
        routed[e] = run;
        kept[e] = kv;
        kept_s[e] = kv;
      }
    }
    lds_barrier();  // part is taken again
  }
  scan_tail(tail, kept_s, kpre, send_s, sh);
}

__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ tile_cnt, int64_t nt,
                                                    int32_t* __restrict__ tile_off, int32_t* __restrict__ routed,
                                                    int32_t* __restrict__ kept, ScanTail tail) {
  extern __shared__ int sm[];
  scan_block<16>(tile_cnt, nt, tile_off, routed, kept, tail, sm);
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

// Slots from the scan and the in-tile ranks. A block of 256 threads takes
// floor(256 / k) whole tokens, one thread per copy: slot = tile_off[tile][e]
// + rank, kept when below C (rank -1 or an expert outside [0, E): dropped).
// slot holds the ranks on entry and the slots on exit (each thread reads its
// entry, then writes it). Also src (kept rows) and, per block, one addition
// of its tokens with no kept copy to totals[1].
__global__ __launch_bounds__(256) void slots_from_ranks_kernel(const int32_t* __restrict__ idx,
                                                               int32_t* __restrict__ slot,
                                                               const int32_t* __restrict__ tile_off, int64_t T,
                                                               int k, int E, int64_t C, int32_t* __restrict__ src,
                                                               int64_t* __restrict__ totals) {
  __shared__ int any[256];
  const int tb = 256 / k;
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tb;
  const int n = static_cast<int>(min<int64_t>(tb, T - t0));
  if (tid < tb) any[tid] = 0;
  lds_barrier();
  if (tid < n * k) {
    const int64_t i = t0 * k + tid;
    const int e = idx[i];
    const int r = slot[i];
    int sl = -1;
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E) && r >= 0) {
      const int64_t v = tile_off[((t0 + tid / k) / kTileTokens) * E + e] + static_cast<int64_t>(r);
      if (v < C) sl = static_cast<int>(v);
    }
    slot[i] = sl;
    if (sl >= 0) {
      any[tid / k] = 1;  // every writer stores the same value
      if (src) src[static_cast<int64_t>(e) * C + sl] = static_cast<int32_t>(i);
    }
  }
  lds_barrier();
  if (totals && tid < 64) {
    int c = 0;
    for (int j = tid; j < n; j += 64) c += any[j] == 0 ? 1 : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
    if (tid == 0 && c) atomicAdd(reinterpret_cast<unsigned long long*>(&totals[1]), static_cast<unsigned long long>(c));
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

// Slots and row scatter in one launch, for layers whose earlier tiles'
// counts are few enough for each block to add up. Block 0 runs the scan
// (counts, totals but totals[1], tile maps, cleared split-K counters); every
// other block takes 1024 / H tokens of one 64-token tile, H threads each, and
// adds up the tile histogram over the earlier tiles itself, so no block waits
// for the scan: slot = that sum for the copy's expert + the copy's rank within
// its tile (held in slot on entry), kept below C, exactly as tile_off + rank.
// With BP (E (nt - 1) <= 65536) the whole block sums every expert's column,
// the first tl E words of the histogram (at most 64 counts a thread, 16 loads
// in flight); otherwise each token's threads sum the column of each copy's
// expert (k (nt - 1) <= 256, one count per thread). The row words (U per lane) are loaded
// first, while the counts are on their way; the copies then go out as in
// scatter_rows_kernel. totals[1] must be zero on entry: each block adds its
// fully dropped tokens once.
template <int U, int H, bool BP>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8, 8))) void slot_scatter_kernel(
    const int32_t* __restrict__ tile_cnt, int64_t nt, int32_t* __restrict__ tile_off, int32_t* __restrict__ routed,
    int32_t* __restrict__ kept, ScanTail tail, const uint4* __restrict__ x, const int32_t* __restrict__ idx,
    int32_t* __restrict__ slot, int32_t* __restrict__ src, int64_t V, uint4* __restrict__ buckets) {
  static_assert(H == 64 || H == 128 || H == 256, "one to four waves per token");
  extern __shared__ int sm[];
  if (blockIdx.x == 0) {
    scan_block<4>(tile_cnt, nt, tile_off, routed, kept, tail, sm);  // short runs: few counts kept
    return;
  }
  constexpr int KM = 32;          // copies per token at most
  constexpr int TB = 1024 / H;    // tokens per block, all of one tile
  constexpr int PI = 256 / H;     // per-copy counts per thread at most
  __shared__ int psum[BP ? 4096 : TB * KM], sls[TB * KM], es[TB * KM], fd[TB];
  const int E = tail.E, k = tail.k;
  const int64_t T = tail.T, C = tail.C;
  const int tid = threadIdx.x;
  const int q = tid / H, u = tid % H, wl = tid & 63;
  const bool first_wave = u < 64;  // of the token's H / 64
  const int64_t t = (static_cast<int64_t>(blockIdx.x) - 1) * TB + q;
  const bool live = t < T;
  const int tl = static_cast<int>(t / kTileTokens);  // earlier tiles: 0 .. tl - 1 (one value per block)
  if constexpr (BP) {
    for (int e = tid; e < E; e += 1024) psum[e] = 0;
  } else {
    if (u < k) psum[q * KM + u] = 0;
  }
  if (u == 0) fd[q] = 0;
  // the copies' experts and ranks (first wave), the row, the prefix operands
  int e0 = -1, r0 = -1;
  if (live && first_wave && wl < k) {
    e0 = idx[t * k + wl];
    r0 = slot[t * k + wl];
  }
  const uint4* xr = x + t * V;
  uint4 val[U];
  if (live) {
#pragma unroll
    for (int w = 0; w < U; ++w) {
      const int64_t v = u + H * w;
      if (v < V) val[w] = xr[v];
    }
  }
  if constexpr (BP) {
    // count c is tile c / E's count of expert c % E; thread i takes counts
    // i, i + 1024, ...: with E a power of two up to 1024 all of one expert,
    // summed in registers; otherwise the expert advances by 1024 mod E a count
    const int npre = E * tl;  // the block's first token is live
    constexpr int B = 16;
    const bool pow2 = (E & (E - 1)) == 0 && E <= 1024;
    const int step = 1024 % E;
    int ex = tid % E;
    int acc = 0;
    lds_barrier();  // psum is zero
    for (int c0 = 0; c0 < npre; c0 += B * 1024) {
      int v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int c = c0 + i * 1024 + tid;
        v[i] = c < npre ? tile_cnt[c] : 0;
      }
      if (pow2) {
#pragma unroll
        for (int i = 0; i < B; ++i) acc += v[i];
      } else {
#pragma unroll
        for (int i = 0; i < B; ++i) {
          if (v[i]) atomicAdd(&psum[ex], v[i]);  // integer sums: any order
          ex += step;
          ex -= ex >= E ? E : 0;
        }
      }
    }
    if (acc) atomicAdd(&psum[tid & (E - 1)], acc);  // pow2 only: acc stays 0 otherwise
  } else {
    const int npre = live ? k * tl : 0;
    int pj[PI], pe[PI], pv[PI];
#pragma unroll
    for (int i = 0; i < PI; ++i) {
      const int c = u + i * H;
      pj[i] = 0;
      pe[i] = -1;
      if (c < npre) {
        pj[i] = c / tl;
        pe[i] = idx[t * k + pj[i]];
      }
    }
#pragma unroll
    for (int i = 0; i < PI; ++i) {
      pv[i] = 0;
      if (static_cast<unsigned>(pe[i]) < static_cast<unsigned>(E))
        pv[i] = tile_cnt[static_cast<int64_t>(u + i * H - pj[i] * tl) * E + pe[i]];
    }
    lds_barrier();  // psum is zero
#pragma unroll
    for (int i = 0; i < PI; ++i)
      if (pv[i]) atomicAdd(&psum[q * KM + pj[i]], pv[i]);  // integer sums: any order
  }
  lds_barrier();
  int sl = -1;
  if (live && first_wave && wl < k) {
    if (static_cast<unsigned>(e0) < static_cast<unsigned>(E) && r0 >= 0) {
      const int64_t v = psum[BP ? e0 : q * KM + wl] + static_cast<int64_t>(r0);
      if (v < C) sl = static_cast<int>(v);
    }
    slot[t * k + wl] = sl;  // this lane read the rank from the same word
    if (sl >= 0 && src) src[static_cast<int64_t>(e0) * C + sl] = static_cast<int32_t>(t * k + wl);
    sls[q * KM + wl] = sl;
    es[q * KM + wl] = e0;
  }
  if (first_wave) {
    const uint64_t any = __ballot(sl >= 0);
    if (live && wl == 0 && any == 0) fd[q] = 1;
  }
  lds_barrier();
  int s_l = -1, e_l = 0;
  if (live && wl < k) {
    s_l = sls[q * KM + wl];
    e_l = es[q * KM + wl];
  }
  const uint64_t keep = __ballot(s_l >= 0);
  if (threadIdx.x == 0 && tail.totals) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < TB; ++i) c += fd[i];
    if (c) atomicAdd(reinterpret_cast<unsigned long long*>(&tail.totals[1]), static_cast<unsigned long long>(c));
  }
  if (!live) return;
  for (int64_t v0 = u; v0 < V; v0 += H * U) {
    if (v0 != u) {
#pragma unroll
      for (int w = 0; w < U; ++w) {
        const int64_t v = v0 + H * w;
        if (v < V) val[w] = xr[v];
      }
    }
    for (uint64_t m = keep; m; m &= m - 1) {
      const int j = __builtin_ctzll(m);
      const int e = __builtin_amdgcn_readlane(e_l, j);
      const int sj = __builtin_amdgcn_readlane(s_l, j);
      uint4* dst = buckets + (static_cast<int64_t>(e) * C + sj) * V;
#pragma unroll
      for (int w = 0; w < U; ++w) {
        const int64_t v = v0 + H * w;
        if (v < V) store_stream(&dst[v], val[w]);
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
  __syncthreads();  // these stores complete before other threads overwrite them (the scan's barriers order LDS only)
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
                            hipStream_t s, int32_t* rank, int64_t* zero) {
  const int64_t nt = ceil_div(T, kTileTokens);
  if (nt == 0) return hipSuccess;
  const size_t shm = (static_cast<size_t>(E) + static_cast<size_t>(kTileTokens) * k +
                     (tile_ranks_by_waves(k, E) ? static_cast<size_t>(k) * E : 0)) * sizeof(int);
  tile_hist_kernel<<<dim3(static_cast<unsigned>(nt)), dim3(1024), shm, s>>>(idx, T, k, E, tile_cnt, rank,
                                                                             zero);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* tile_cnt, int64_t nt, int E, int64_t C, int P,
                       int64_t row_bytes, int k, int64_t T, int32_t* tile_off, int32_t* routed,
                       int32_t* kept, int32_t* send, int64_t* totals, int bm, int32_t* mtile_off,
                       int32_t* src, hipStream_t s, const int32_t* place, int bm1, int32_t* mtile1,
                       int32_t* clear, int n_clear) {
  if (E > 4096 || P < 1 || P > E || nt * E >= (int64_t{1} << 31) || n_clear < 0) return hipErrorInvalidValue;
  const ScanTail tail{C, row_bytes, T, E, P, k, send, totals, bm, bm1, mtile_off, mtile1, place, clear, n_clear};
  const size_t shm = (2 * static_cast<size_t>(E) + 1 + P) * sizeof(int);
  scan_kernel<<<dim3(1), dim3(1024), shm, s>>>(tile_cnt, nt, tile_off, routed, kept, tail);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !src) return err;
  const unsigned gx = static_cast<unsigned>(std::min<int64_t>(ceil_div(C, 256), 64));
  src_padding_kernel<<<dim3(gx, static_cast<unsigned>(E)), dim3(256), 0, s>>>(kept, C, E, src);
  return hipGetLastError();
}

hipError_t launch_slots_from_ranks(const int32_t* idx, int32_t* slot, const int32_t* tile_off, int64_t T, int k,
                                  int E, int64_t C, int32_t* src, int64_t* totals, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k < 1 || k > 256) return hipErrorInvalidValue;
  const int tb = 256 / k;
  slots_from_ranks_kernel<<<dim3(static_cast<unsigned>(ceil_div(T, tb))), dim3(256), 0, s>>>(idx, slot, tile_off, T,
                                                                                             k, E, C, src, totals);
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

namespace {
// each block of the one-pass kernel sums every expert's column of the earlier tiles
bool slot_scatter_block_prefix(int64_t nt, int E) { return E <= 4096 && (nt - 1) * E <= 65536; }
}  // namespace

bool slot_scatter_fits(int64_t T, int k, int E) {
  const int64_t nt = ceil_div(T, kTileTokens);
  return T > 0 && k <= 32 && E <= 4096 && ((nt - 1) * k <= 256 || slot_scatter_block_prefix(nt, E));
}

hipError_t launch_slot_scatter(const int32_t* tile_cnt, int E, int64_t C, int P, int64_t row_bytes, int k,
                               int64_t T, int32_t* tile_off, int32_t* routed, int32_t* kept, int32_t* send,
                               int64_t* totals, int bm, int32_t* mtile_off, int bm1, int32_t* mtile1,
                               int32_t* clear, int n_clear, const void* x, const int32_t* idx, int32_t* slot,
                               int32_t* src, void* buckets, hipStream_t s, const int32_t* place) {
  if (!slot_scatter_fits(T, k, E) || P < 1 || P > E || n_clear < 0) return hipErrorInvalidValue;
  const int64_t nt = ceil_div(T, kTileTokens);
  ScanTail tail{C, row_bytes, T, E, P, k, send, totals, bm, bm1, mtile_off, mtile1, place, clear, n_clear};
  tail.leave_t1 = true;
  const size_t shm = (2 * static_cast<size_t>(E) + 1 + P) * sizeof(int);
  const auto* xv = static_cast<const uint4*>(x);
  auto* bv = static_cast<uint4*>(buckets);
  const int64_t V = row_bytes / 16;
  // threads per token: the fewest of 64, 128, 256 that cover the row with four
  // words a lane (one word for rows of at most 64), 256 with eight beyond 1024
  const bool bp = slot_scatter_block_prefix(nt, E);
  auto go = [&](auto u_c, auto h_c) {
    constexpr int U = decltype(u_c)::value, H = decltype(h_c)::value;
    const dim3 grid(static_cast<unsigned>(1 + ceil_div(T, 1024 / H)));
    if (bp)
      slot_scatter_kernel<U, H, true><<<grid, dim3(1024), shm, s>>>(tile_cnt, nt, tile_off, routed, kept, tail, xv,
                                                                    idx, slot, src, V, bv);
    else
      slot_scatter_kernel<U, H, false><<<grid, dim3(1024), shm, s>>>(tile_cnt, nt, tile_off, routed, kept, tail, xv,
                                                                     idx, slot, src, V, bv);
  };
  using I1 = std::integral_constant<int, 1>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  if (V <= 64)
    go(I1{}, std::integral_constant<int, 64>{});
  else if (V <= 256)
    go(I4{}, std::integral_constant<int, 64>{});
  else if (V <= 512)
    go(I4{}, std::integral_constant<int, 128>{});
  else if (V <= 1024)
    go(I4{}, std::integral_constant<int, 256>{});
  else
    go(I8{}, std::integral_constant<int, 256>{});
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !src) return err;
  const unsigned gx = static_cast<unsigned>(std::min<int64_t>(ceil_div(C, 256), 64));
  src_padding_kernel<<<dim3(gx, static_cast<unsigned>(E)), dim3(256), 0, s>>>(kept, C, E, src);
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
