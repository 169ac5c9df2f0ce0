// Router of the MoE layer: scores, top-k choice and gate weights (gfx950).
//
// Sources: "Expert Parallelism" (klaylearn.com glossary) - the router scores
// each token against every expert, keeps the top k and yields the weights
// that combine their outputs; "Expert Parallelism" (inferensys.com glossary),
// gating-network entry - a small linear router with top-k gating.
//
// logits[t, e] = sum_i x[t, i] W_router[e, i] (+ bias[e]), fp32.
// Top-k: order by score descending, then expert index ascending (the pages
// leave ties open; the lower index wins). Gates: softmax over the k chosen
// scores, evaluated in fp64 and rounded to fp32.
#include <algorithm>
#include <climits>

#include "common.h"

namespace moe {
namespace {

constexpr int kMaxRouterSplits = 16;  // d-slices of the router scores (partials summed in order)
constexpr int kTiledSplits = 8;       // at most this many when a wave takes 2 or 4 token tiles
// With this many experts or more and fewer 64-token tiles than kWideRouteTiles
// (decode-sized batches), top-k takes a whole wave per token (16 tokens a
// block, four times the blocks of 16-lane groups) and the tile histogram and
// ranks come from the tile kernel that follows: the DeepSeek-V3 decode route
// 39 -> 16 + 5 us. With 128 tiles (DeepSeek-V3 prefill) it measured even.
constexpr int kWideRouteE = 128, kWideRouteTiles = 64;

// ---------------------------------------------------------------------------
// Scores on the matrix cores. Each wave is one work item: 16 MT tokens x
// (16 NT) experts over one of S slices of d, with v_mfma_f32_16x16x32_bf16;
// each router-weight fragment it loads serves its MT token tiles. It writes
// fp32 partial sums part[s][t][e]. The route kernel adds the S partials in
// slice order (a fixed order: the result does not depend on scheduling), so
// few tokens still spread over many waves. Both operands come straight from
// global memory (x is read once; W_router is small and stays in L2).
// Lane l of an A/B operand holds row (l % 16), K elements 8*(l/16) .. +8;
// the accumulator of lane l holds rows 4*(l/16) + r, column l % 16.
// ---------------------------------------------------------------------------
template <int NT, int MT>
__global__ __launch_bounds__(256) void router_logits_bf16(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wr, int64_t T,
                                                          int64_t d, int E, int S, int64_t kper,
                                                          float* __restrict__ part) {
  constexpr int U = MT <= 2 ? 4 : 2;  // k-steps whose loads are in flight together
  const int lane = threadIdx.x & 63;
  const int64_t tt = ceil_div(T, 16 * MT);
  const int64_t ec = ceil_div(E, 16 * NT);
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (item >= tt * ec * S) return;
  const int64_t t0 = (item % tt) * 16 * MT;
  const int e0 = static_cast<int>((item / tt) % ec) * 16 * NT;
  const int s = static_cast<int>(item / (tt * ec));
  const int64_t k_lo = s * kper, k_hi = min(d, k_lo + kper);
  const int kg = (lane >> 4) * 8;
  const bf16_t* xp[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t trow = min(t0 + 16 * m + (lane & 15), T - 1);  // rows past T are computed, not stored
    xp[m] = x + trow * d + kg;
  }
  const bf16_t* wp[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int e = min(e0 + 16 * j + (lane & 15), E - 1);
    wp[j] = wr + static_cast<int64_t>(e) * d + kg;
  }
  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  int64_t k0 = k_lo;
  for (; k0 + U * 32 <= k_hi; k0 += U * 32) {
    bf16x8 a[U][MT], b[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int m = 0; m < MT; ++m) a[u][m] = *reinterpret_cast<const bf16x8*>(xp[m] + k0 + 32 * u);
#pragma unroll
      for (int j = 0; j < NT; ++j) b[u][j] = *reinterpret_cast<const bf16x8*>(wp[j] + k0 + 32 * u);
    }
    // every load of the group goes out before the first product (left to
    // itself the scheduler interleaves them, keeping about two k-steps in
    // flight: 12.0 -> 11.0 us on T = 4096, d = 4096, E = 8 with U = 4)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][m], b[u][j], acc[m][j], 0, 0, 0);
  }
  for (; k0 < k_hi; k0 += 32) {
    const bool in = k0 + kg < k_hi;  // d is a multiple of 8: whole 8-element groups
    bf16x8 a[MT], b[NT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      a[m] = bf16x8{};
      if (in) a[m] = *reinterpret_cast<const bf16x8*>(xp[m] + k0);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      b[j] = bf16x8{};
      if (in) b[j] = *reinterpret_cast<const bf16x8*>(wp[j] + k0);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b[j], acc[m][j], 0, 0, 0);
  }
  float* ps = part + static_cast<int64_t>(s) * T * E;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int e = e0 + 16 * j + (lane & 15);
      if (e >= E) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 16 * m + 4 * (lane >> 4) + r;
        if (t < T) ps[t * E + e] = acc[m][j][r];
      }
    }
}

// fp32 scores: one thread per (token, expert), plain fused multiply-adds.
__global__ __launch_bounds__(256) void router_logits_f32(const float* __restrict__ x,
                                                         const float* __restrict__ wr, int64_t T,
                                                         int64_t d, int E, float* __restrict__ part) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= T * E) return;
  const int64_t t = i / E;
  const int e = static_cast<int>(i % E);
  const float* xr = x + t * d;
  const float* wrow = wr + static_cast<int64_t>(e) * d;
  float acc = 0.f;
  for (int64_t c = 0; c < d; ++c) acc = fmaf(xr[c], wrow[c], acc);
  part[i] = acc;
}

// ---------------------------------------------------------------------------
// Top-k and gates. A group of L lanes serves one token: lane g keeps a sorted
// list of its best KMAX scores among experts g, g+L, ...; then k rounds pick
// the group's best head (score desc, index asc) with a butterfly reduction and
// pop it from its owner. Lane j < k of the group ends with the j-th choice.
//
// Rank-limited variant (LIMIT): "Expert Parallelism & All-to-All"
// (neelmishra.github.io), "The bandwidth bill" - node-limited routing keeps a
// token's experts on a few nodes; "Expert parallelism vs tensor parallelism for
// MoE" (fanout.sh), "Expert parallelism pays in all-to-all dispatch" - at most
// 4 nodes per token in DeepSeek-V3. Rank p owns experts [p E/P, (p+1) E/P); a
// rank's score is its best expert score; the M best ranks (lower index on a
// tie) are allowed and the top k is taken over their experts only. Pass 1 sums
// the scores, keeps them (in lsum, or where they already are) and folds each
// into its rank's best with an order-preserving integer max in LDS; pass 2
// ranks the P ranks; pass 3 is the plain top-k over the allowed experts.
// ---------------------------------------------------------------------------
constexpr int kMaxLimitRanks = 64;  // P limit of the rank-limited variant (one 64-bit mask)

__device__ inline bool better(float v, int e, float ov, int oe) {
  return v > ov || (v == ov && e < oe);
}

// Monotone map of a float (not NaN) to uint32: a < b  <=>  key(a) < key(b).
__device__ inline uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// SEL: selects instead of a masked branch per slot. With many scores a lane
// (DeepSeek-V3 prefill: 16 of 256) the branches took most of the route
// kernel's time (39 -> 30 us with selects); with few (4 a lane on the skewed
// and decode shapes) the branches, mostly skipped, are cheaper (19.2 -> 20.4
// us and 18.2 -> 20.6 us with selects). The route launch picks SEL from the
// scores per lane.
template <int KMAX, bool SEL>
__device__ inline void insert_sorted(float (&lv)[KMAX], int (&li)[KMAX], float v, int ei) {
  bool ins = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool take = ins || better(v, ei, lv[j], li[j]);  // from here on every entry moves down one
    if constexpr (SEL) {
      const float tv = lv[j];
      const int te = li[j];
      lv[j] = take ? v : tv;
      li[j] = take ? ei : te;
      v = take ? tv : v;
      ei = take ? te : ei;
    } else if (take) {
      const float tv = lv[j];
      const int te = li[j];
      lv[j] = v;
      li[j] = ei;
      v = tv;
      ei = te;
    }
    ins = take;
  }
}

template <int L, int KMAX, bool HIST, bool LIMIT, bool SEL>
__global__ __launch_bounds__(1024) void route_kernel(const float* part, int S, const float* __restrict__ bias,
                                                     int64_t T, int E, int k, float* logits_out,
                                                     int32_t* __restrict__ idx, float* __restrict__ w,
                                                     int32_t* __restrict__ tile_cnt, int P, int M,
                                                     float* lsum, const float* lsrc, int32_t* __restrict__ rank,
                                                     int64_t* zero) {
  constexpr int kTokensPerBlock = 1024 / L;
  static_assert(!HIST || kTokensPerBlock == kTileTokens, "one block per histogram tile");
  extern __shared__ int smem[];
  int* hist = smem;                                                            // [E] when HIST
  uint32_t* rbest = reinterpret_cast<uint32_t*>(smem + (HIST ? E : 0));        // [tokens][P] when LIMIT
  int* ecp = smem + (HIST ? E : 0) + (LIMIT ? kTokensPerBlock * P : 0);        // [tokens][k] when HIST
  const int g = threadIdx.x % L;
  const int tok = threadIdx.x / L;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + tok;
  const bool valid = t < T;
  if (zero && blockIdx.x == 0 && threadIdx.x == 0) *zero = 0;
  if (HIST)
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  if (LIMIT)
    for (int i = threadIdx.x; i < kTokensPerBlock * P; i += blockDim.x) rbest[i] = 0u;  // below every key
  if (HIST || LIMIT) __syncthreads();
  const int per = LIMIT ? E / P : 1;  // experts per rank

  float lv[KMAX];
  int li[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    lv[j] = -INFINITY;
    li[j] = INT_MAX;
  }
  if (valid) {
    const int64_t TE = T * E;
    constexpr int G = 4;  // experts whose scores are fetched together (loads in flight)
    for (int eb = g; eb < E; eb += G * L) {
      float vv[G];
#pragma unroll
      for (int q = 0; q < G; ++q) {
        const int e = eb + q * L;
        vv[q] = e < E ? part[t * E + e] : 0.f;
      }
      for (int s0 = 1; s0 < S; s0 += 8) {
        float pv[8][G];  // eight slices' loads in flight at once
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int q = 0; q < G; ++q) {
            const int e = eb + q * L;
            pv[j][q] = (s0 + j < S && e < E) ? part[(s0 + j) * TE + t * E + e] : 0.f;
          }
#pragma unroll
        for (int j = 0; j < 8; ++j)  // slice order
#pragma unroll
          for (int q = 0; q < G; ++q)
            if (s0 + j < S) vv[q] += pv[j][q];
      }
#pragma unroll
      for (int q = 0; q < G; ++q) {
        const int e = eb + q * L;
        if (e >= E) break;
        float v = vv[q];
        if (bias) v += bias[e];
        if (logits_out) logits_out[t * E + e] = v;
        v += 0.0f;  // -0.0 -> +0.0 (they compare equal anyway)
        if (LIMIT) {
          if (lsum) lsum[t * E + e] = v;
          atomicMax(&rbest[tok * P + e / per], order_key(v));
        } else {
          insert_sorted<KMAX, SEL>(lv, li, v, e);
        }
      }
    }
  }

  if (LIMIT) {
    __syncthreads();  // every rank's best is in LDS
    uint64_t allowed = 0;
    const uint32_t* rb = rbest + tok * P;
    for (int p = g; p < P; p += L) {
      const uint32_t kp = rb[p];
      int pos = 0;  // ranks ahead of p: better score, or equal score and lower index
      for (int q = 0; q < P; ++q) {
        const uint32_t kq = rb[q];
        pos += (kq > kp || (kq == kp && q < p)) ? 1 : 0;
      }
      if (pos < M) allowed |= uint64_t{1} << p;
    }
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1) {
      const uint32_t lo = __shfl_xor(static_cast<uint32_t>(allowed), off, L);
      const uint32_t hi = __shfl_xor(static_cast<uint32_t>(allowed >> 32), off, L);
      allowed |= (static_cast<uint64_t>(hi) << 32) | lo;
    }
    if (valid) {
      constexpr int G = 4;
      for (int eb = g; eb < E; eb += G * L) {
        float vv[G];
#pragma unroll
        for (int q = 0; q < G; ++q) {
          const int e = eb + q * L;
          vv[q] = e < E ? lsrc[t * E + e] : 0.f;  // written by this lane in pass 1, or an input
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
          const int e = eb + q * L;
          if (e >= E) break;
          if ((allowed >> (e / per)) & 1u) insert_sorted<KMAX, SEL>(lv, li, vv[q] + 0.0f, e);
        }
      }
    }
  }

  float sel_v = -INFINITY, v0 = 0.f;
  int sel_e = 0;
  for (int r = 0; r < k; ++r) {
    float bv = lv[0];
    int be = li[0];
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, L);
      const int oe = __shfl_xor(be, off, L);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if (r == 0) v0 = bv;
    if (g == r) {
      sel_v = bv;
      sel_e = be;
    }
    const bool pop = li[0] == be;  // the owner pops its head
    if constexpr (SEL) {
#pragma unroll
      for (int j = 0; j + 1 < KMAX; ++j) {
        lv[j] = pop ? lv[j + 1] : lv[j];
        li[j] = pop ? li[j + 1] : li[j];
      }
      lv[KMAX - 1] = pop ? -INFINITY : lv[KMAX - 1];
      li[KMAX - 1] = pop ? INT_MAX : li[KMAX - 1];
    } else if (pop) {
#pragma unroll
      for (int j = 0; j + 1 < KMAX; ++j) {
        lv[j] = lv[j + 1];
        li[j] = li[j + 1];
      }
      lv[KMAX - 1] = -INFINITY;
      li[KMAX - 1] = INT_MAX;
    }
  }

  const double z = g < k ? exp(static_cast<double>(sel_v) - static_cast<double>(v0)) : 0.0;
  double sum = z;
#pragma unroll
  for (int off = L / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, L);
  sum = __shfl(sum, 0, L);  // one denominator for the whole group
  if (valid && g < k) {
    idx[t * k + g] = sel_e;
    w[t * k + g] = static_cast<float>(z / sum);
  }
  if (HIST) {  // the tile's histogram and the ranks of its copies
    if (g < k) ecp[tok * k + g] = sel_e;
    lds_barrier();
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock;
    const int ncp = static_cast<int>(min<int64_t>(kTokensPerBlock, T - t0)) * k;
    int32_t* rk = rank ? rank + t0 * k : nullptr;
    if (tile_ranks_by_waves(k, E)) {
      rank_tile_waves(ecp, ncp, E, hist, ecp + kTokensPerBlock * k, rk);
    } else {
      if (threadIdx.x < 64) rank_tile(ecp, ncp, E, hist, rk);
      lds_barrier();
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) tile_cnt[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
  }
}

struct RouteArgs {
  const float* part;
  int S;
  const float* bias;
  int64_t T;
  int E, k;
  float* logits_out;
  int32_t* idx;
  float* w;
  int32_t* tile_cnt;
  int P, M;
  float* lsum;
  const float* lsrc;
  int32_t* rank;
  int64_t* zero;
};

template <int L, int KMAX, bool HIST, bool LIMIT>
hipError_t route_launch(const RouteArgs& a, hipStream_t s) {
  const bool sel = a.E >= 8 * L;  // eight or more scores a lane: selects in the top-k insertion
  const int64_t tpb = 1024 / L;
  // HIST: histogram [E], the tile's experts [64 k] and, for the ranking by all waves, its chunk counts [k E]
  const size_t lds = (HIST ? (a.E + tpb * a.k + (tile_ranks_by_waves(a.k, a.E) ? a.k * a.E : 0)) * sizeof(int) : 0) +
                     (LIMIT ? tpb * a.P * sizeof(uint32_t) : 0);
  const dim3 grid(static_cast<unsigned>(ceil_div(a.T, tpb)));
  if (sel)
    route_kernel<L, KMAX, HIST, LIMIT, true><<<grid, dim3(1024), lds, s>>>(
        a.part, a.S, a.bias, a.T, a.E, a.k, a.logits_out, a.idx, a.w, a.tile_cnt, a.P, a.M, a.lsum, a.lsrc, a.rank,
        a.zero);
  else
    route_kernel<L, KMAX, HIST, LIMIT, false><<<grid, dim3(1024), lds, s>>>(
        a.part, a.S, a.bias, a.T, a.E, a.k, a.logits_out, a.idx, a.w, a.tile_cnt, a.P, a.M, a.lsum, a.lsrc, a.rank,
        a.zero);
  return hipGetLastError();
}

template <bool LIMIT>
hipError_t route_dispatch(const RouteArgs& a, hipStream_t s) {
  if (a.tile_cnt) {
    if (a.k <= 2) return route_launch<16, 2, true, LIMIT>(a, s);
    if (a.k <= 8) return route_launch<16, 8, true, LIMIT>(a, s);
    return route_launch<16, 16, true, LIMIT>(a, s);
  }
  if (a.E >= kWideRouteE && a.k <= 16 && ceil_div(a.T, kTileTokens) < kWideRouteTiles) {  // a wave per token
    if (a.k <= 2) return route_launch<64, 2, false, LIMIT>(a, s);
    if (a.k <= 8) return route_launch<64, 8, false, LIMIT>(a, s);
    return route_launch<64, 16, false, LIMIT>(a, s);
  }
  if (a.k <= 2) return route_launch<16, 2, false, LIMIT>(a, s);
  if (a.k <= 8) return route_launch<16, 8, false, LIMIT>(a, s);
  if (a.k <= 16) return route_launch<16, 16, false, LIMIT>(a, s);
  return route_launch<32, 32, false, LIMIT>(a, s);
}

}  // namespace

// With many experts the score GEMM is a real one (T x E x d): it runs on the
// grouped GEMM's 256 x 256 LDS-DMA tiles with fp32 output, so each tile of
// router weights is read once per 256 tokens, not once per 16. (With fewer
// than 128 experts most of a 256-wide tile would be padding.)
// The GEMM kernel addresses x as one buffer of 32-bit byte offsets, so x must
// stay below 2^31 bytes there; larger batches keep the wave kernel.
static bool router_on_gemm(int64_t T, int64_t d, int E, bool bf16) {
  return bf16 && E >= 128 && E % 8 == 0 && T >= 256 && d % 128 == 0 && T * d * 2 < (int64_t{1} << 31);
}

// Token tiles of 16 per wave of the score kernel: the largest of 4 and 2 that
// still gives 1024 waves with the most d-slices allowed, else 1. Each router
// weight fragment a wave loads then serves that many tiles (measured on
// T = 16384, E = 64: 43 -> 26 us; T = 4096, E = 8: 10.7 -> 10.0 us).
static int router_tile_tokens(int64_t T, int64_t d, int E) {
  const int nt = E <= 16 ? 1 : (E <= 32 ? 2 : 4);
  const int64_t s_max = std::max<int64_t>(1, std::min<int64_t>(d / 256, kTiledSplits));
  for (int mt : {4, 2})
    if (ceil_div(T, 16 * mt) * ceil_div(E, 16 * nt) * s_max >= 1024) return mt;
  return 1;
}

int router_splits(int64_t T, int64_t d, int E, bool bf16) {
  if (!bf16 || T == 0) return 1;
  if (router_on_gemm(T, d, E, bf16)) {  // d-slices so that about 256 tiles run at once
    const int64_t tiles = ceil_div(T, 256) * ceil_div(E, 256);
    return static_cast<int>(std::max<int64_t>(
        1, std::min({ceil_div(256, tiles), d / 128, int64_t{kMaxRouterSplits}})));
  }
  const int nt = E <= 16 ? 1 : (E <= 32 ? 2 : 4);
  const int mt = router_tile_tokens(T, d, E);
  const int64_t items = ceil_div(T, 16 * mt) * ceil_div(E, 16 * nt);
  const int64_t by_work = ceil_div(mt == 1 ? 2048 : 1024, items);  // aim at >= 2048 (1024) waves
  const int64_t by_len = std::max<int64_t>(1, d / 256);              // at least 256 of d per slice
  const int64_t cap = mt == 1 ? kMaxRouterSplits : kTiledSplits;   // few tokens: more slices
  return static_cast<int>(std::max<int64_t>(1, std::min({by_work, by_len, cap})));
}

hipError_t launch_router_logits(const void* x, const void* wr, int64_t T, int64_t d, int E, bool bf16,
                                int S, float* part, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (router_on_gemm(T, d, E, bf16)) return launch_gemm_rows_f32(x, wr, T, d, E, S, part, s);
  if (!bf16) {
    const int64_t n = T * E;
    router_logits_f32<<<dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s>>>(
        static_cast<const float*>(x), static_cast<const float*>(wr), T, d, E, part);
    return hipGetLastError();
  }
  const int nt = E <= 16 ? 1 : (E <= 32 ? 2 : 4);
  const int mt = router_tile_tokens(T, d, E);
  const int64_t kper = ceil_div(ceil_div(d, S), 32) * 32;
  const int64_t items = ceil_div(T, 16 * mt) * ceil_div(E, 16 * nt) * S;
  const dim3 grid(static_cast<unsigned>(ceil_div(items, 4)));
  const auto* xb = static_cast<const bf16_t*>(x);
  const auto* wb = static_cast<const bf16_t*>(wr);
#define MOE_SCORES(N, M) router_logits_bf16<N, M><<<grid, dim3(256), 0, s>>>(xb, wb, T, d, E, S, kper, part)
#define MOE_SCORES_M(N)                    \
  if (mt == 4)                             \
    MOE_SCORES(N, 4);                      \
  else if (mt == 2)                        \
    MOE_SCORES(N, 2);                      \
  else                                     \
    MOE_SCORES(N, 1)
  if (nt == 1) {
    MOE_SCORES_M(1);
  } else if (nt == 2) {
    MOE_SCORES_M(2);
  } else {
    MOE_SCORES_M(4);
  }
#undef MOE_SCORES_M
#undef MOE_SCORES
  return hipGetLastError();
}

bool route_builds_histogram(int k, int E, int64_t T) {
  return k <= 16 && (E < kWideRouteE || ceil_div(T, kTileTokens) >= kWideRouteTiles);
}

bool route_rank_limited(int P, int M) { return M > 0 && M < P; }

hipError_t launch_route(const float* part, int S, const float* bias, int64_t T, int E, int k,
                        float* logits_out, int32_t* idx, float* w, int32_t* tile_cnt, int P, int M,
                        hipStream_t s, int32_t* rank, int64_t* zero) {
  if (T == 0) return hipSuccess;
  if (tile_cnt && !route_builds_histogram(k, E, T)) return hipErrorInvalidValue;
  RouteArgs a{part, S, bias, T, E, k, logits_out, idx, w, tile_cnt, P, M, nullptr, nullptr, rank, zero};
  if (!route_rank_limited(P, M)) return route_dispatch<false>(a, s);
  if (P > kMaxLimitRanks || E % P || static_cast<int64_t>(M) * (E / P) < k) return hipErrorInvalidValue;
  // Where pass 3 finds the summed scores: logits_out when asked for, the single
  // unbiased slice itself, else written back over slice 0 (workspace).
  if (logits_out) {
    a.lsrc = logits_out;
  } else if (S == 1 && !bias) {
    a.lsrc = part;
  } else {
    a.lsum = const_cast<float*>(part);
    a.lsrc = part;
  }
  return route_dispatch<true>(a, s);
}

}  // namespace moe
