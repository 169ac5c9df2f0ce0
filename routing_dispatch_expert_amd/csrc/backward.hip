// Backward pass of the MoE layer (gfx950): the row kernels and transposes
// around the grouped GEMMs.
//
// Sources: "Expert Parallelism & All-to-All" (neelmishra.github.io), "The
// bandwidth bill" - the backward pass runs the dispatch and the combine again,
// in reverse; "All-to-all: the distributed transpose" - the combine is the
// exact inverse permutation, weighted by the gates. The gradients are the
// chain rule through the forward, with the top-k choice and the capacity
// drops held fixed (both are piecewise constant):
//
//   combine:  dw[t,j] = <dout[t], y[e,s]> (kept copy (t,j) at expert e, row s),
//             dy[e,s] = w[t,j] dout[t]; a dropped copy has dw = 0
//   gates:    dl[t,j] = w[t,j] (dw[t,j] - sum_i w[t,i] dw[t,i])
//   experts:  h = silu(g) u; dg = dh u silu'(g), du = dh silu(g),
//             silu'(g) = s (1 + g (1 - s)), s = sigmoid(g)
//   dispatch: dx[t] = dout[t] + sum_j [kept] dX[e,s] + sum_j dl[t,j] Wr[e]
//   router:   dWr[e] = sum_t dl[t,e] x[t]; db[e] = sum_t dl[t,e]
//
// Every sum is fp32 in a fixed order; each result is rounded once.
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

// 16-byte words: 8 bf16 or 4 fp32 values.
template <bool BF16>
struct Word {
  static constexpr int N = BF16 ? 8 : 4;
  __device__ static void load(const uint4& v, float (&f)[N]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (BF16) {
        f[2 * q] = __uint_as_float(w[q] << 16);
        f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      } else {
        f[q] = __uint_as_float(w[q]);
      }
    }
  }
  __device__ static uint4 store(const float (&f)[N]) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (BF16)
        w[q] = static_cast<uint32_t>(f32_to_bf16(f[2 * q])) | (static_cast<uint32_t>(f32_to_bf16(f[2 * q + 1])) << 16);
      else
        w[q] = __float_as_uint(f[q]);
    }
    return uint4{w[0], w[1], w[2], w[3]};
  }
};

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Tiled transpose through LDS: dst[b][c][col_off + r] = src[b][r][c] for
// r < valid[b] (all R rows when valid is NULL), and 0 for the other r < Rp;
// src rows are src_ld elements apart, dst rows dst_ld.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t R,
                                                        int64_t Cc, int64_t src_ld, int64_t dst_ld, int64_t col_off,
                                                        int64_t Rp, const int32_t* __restrict__ valid,
                                                        int64_t src_bstride, int64_t dst_bstride) {
  __shared__ T tile[64][65];
  const int64_t b = blockIdx.z;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64, c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t nv = valid ? min(static_cast<int64_t>(valid[b]), R) : R;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const T* s = src + b * src_bstride;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < nv && c < Cc) ? s[r * src_ld + c] : T(0);
  }
  __syncthreads();
  T* d = dst + b * dst_bstride;
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < Cc && r < Rp) d[c * dst_ld + col_off + r] = tile[tx][i];
  }
}

// The same for 2-byte elements in 16-byte words: a 64 x 64 tile comes in as
// row chunks of 8 elements and leaves as chunks of 8 consecutive source rows
// of one column. In LDS, chunk ch of row r sits at position ch ^ (r / 8 % 8),
// so the 16 lanes that read one column for 8 row groups hit distinct banks.
// Needs Cc, src_ld, dst_ld, col_off, Rp and both batch strides multiples of 8
// and 16-byte aligned bases.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                          int64_t R, int64_t Cc, int64_t src_ld, int64_t dst_ld,
                                                          int64_t col_off, int64_t Rp,
                                                          const int32_t* __restrict__ valid, int64_t src_bstride,
                                                          int64_t dst_bstride) {
  __shared__ uint4 tile[64 * 8];
  const int64_t b = blockIdx.z;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64, c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t nv = valid ? min(static_cast<int64_t>(valid[b]), R) : R;
  const int t = threadIdx.x;
  const uint16_t* s = src + b * src_bstride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = t / 8 + 32 * i, ch = t % 8;
    const int64_t gr = r0 + r, gc = c0 + ch * 8;
    uint4 v = {0u, 0u, 0u, 0u};
    if (gr < nv && gc < Cc) v = *reinterpret_cast<const uint4*>(s + gr * src_ld + gc);
    tile[r * 8 + (ch ^ ((r >> 3) & 7))] = v;
  }
  __syncthreads();
  const auto* t16 = reinterpret_cast<const uint16_t*>(tile);
  uint16_t* d = dst + b * dst_bstride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = t / 8 + 32 * i, r8 = t % 8;
    const int64_t gc = c0 + c, gr = r0 + r8 * 8;
    if (gc >= Cc || gr >= Rp) continue;
    const int pos = ((c >> 3) ^ r8) * 8 + (c & 7);  // element c of rows r8 * 8 .. r8 * 8 + 7
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = static_cast<uint32_t>(t16[(r8 * 8 + 2 * q) * 64 + pos]) |
             (static_cast<uint32_t>(t16[(r8 * 8 + 2 * q + 1) * 64 + pos]) << 16);
    *reinterpret_cast<uint4*>(d + gc * dst_ld + col_off + gr) = uint4{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------------------
// SwiGLU on the kept rows of [E][C][F]: forward h = silu(g) u; backward
// dgu[.][0:F] = dh u silu'(g), dgu[.][F:2F] = dh silu(g). One block per row.
// ---------------------------------------------------------------------------
__device__ inline float sigmoidf_(float g) { return 1.0f / (1.0f + expf(-g)); }

template <bool BF16>
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint4* __restrict__ g, const uint4* __restrict__ u,
                                                         uint4* __restrict__ h, const int32_t* __restrict__ kept,
                                                         int64_t C, int64_t VF) {
  const int64_t row = blockIdx.x;
  if (row % C >= kept[row / C]) return;
  using W = Word<BF16>;
  for (int64_t v = threadIdx.x; v < VF; v += blockDim.x) {
    float gf[W::N], uf[W::N], hf[W::N];
    W::load(g[row * VF + v], gf);
    W::load(u[row * VF + v], uf);
#pragma unroll
    for (int q = 0; q < W::N; ++q) hf[q] = gf[q] * sigmoidf_(gf[q]) * uf[q];
    h[row * VF + v] = W::store(hf);
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint4* __restrict__ dh, const uint4* __restrict__ g,
                                                         const uint4* __restrict__ u, uint4* __restrict__ dgu,
                                                         const int32_t* __restrict__ kept, int64_t C, int64_t VF) {
  const int64_t row = blockIdx.x;
  if (row % C >= kept[row / C]) return;
  using W = Word<BF16>;
  for (int64_t v = threadIdx.x; v < VF; v += blockDim.x) {
    float df[W::N], gf[W::N], uf[W::N], dgf[W::N], duf[W::N];
    W::load(dh[row * VF + v], df);
    W::load(g[row * VF + v], gf);
    W::load(u[row * VF + v], uf);
#pragma unroll
    for (int q = 0; q < W::N; ++q) {
      const float s = sigmoidf_(gf[q]);
      dgf[q] = df[q] * uf[q] * s * (1.0f + gf[q] * (1.0f - s));
      duf[q] = df[q] * gf[q] * s;
    }
    dgu[row * 2 * VF + v] = W::store(dgf);
    dgu[row * 2 * VF + VF + v] = W::store(duf);
  }
}

// ---------------------------------------------------------------------------
// Combine backward, one wave per token: dy_j = w_j dout for each kept copy j
// and, with DOT, the dot product dw_j = <dout, y_j> (per-lane partials in
// word order, then a fixed butterfly) and the gate gradients dl.
// ---------------------------------------------------------------------------
template <bool BF16, bool DOT = true>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint4* __restrict__ dout, const uint4* __restrict__ y,
                                                          const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                          const int32_t* __restrict__ slot, int64_t T, int k, int64_t C,
                                                          int64_t V, uint4* __restrict__ dy, float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves only; no barriers below
  using W = Word<BF16>;
  const uint4* drow = dout + t * V;
  if constexpr (!DOT) {
    // dout is read once: U words per lane at a time, then written scaled to
    // every kept copy (non-temporal: nothing here reads them again)
    constexpr int U = 4;
    for (int64_t v0 = 0; v0 < V; v0 += 64 * U) {
      float df[U][W::N];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        if (v < V) W::load(load_stream(drow + v), df[u]);
      }
      for (int j = 0; j < k; ++j) {
        const int sl = __builtin_amdgcn_readfirstlane(slot[t * k + j]);
        if (sl < 0) continue;
        const int64_t base = (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(idx[t * k + j])) * C + sl) * V;
        const float wj = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w[t * k + j])));
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + u * 64 + lane;
          if (v < V) {
            float of[W::N];
#pragma unroll
            for (int q = 0; q < W::N; ++q) of[q] = wj * df[u][q];
            store_stream(dy + base + v, W::store(of));
          }
        }
      }
    }
    return;
  }
  float my_dw = 0.f;  // lane j keeps dw of copy j
  for (int j = 0; j < k; ++j) {
    const int sl = __builtin_amdgcn_readfirstlane(slot[t * k + j]);
    float part = 0.f;
    if (sl >= 0) {
      const int64_t base = (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(idx[t * k + j])) * C + sl) * V;
      const float wj = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w[t * k + j])));
      for (int64_t v = lane; v < V; v += 64) {
        float df[W::N], yf[W::N], of[W::N];
        W::load(drow[v], df);
        if (DOT) W::load(y[base + v], yf);
#pragma unroll
        for (int q = 0; q < W::N; ++q) {
          if (DOT) part = fmaf(df[q], yf[q], part);
          of[q] = wj * df[q];
        }
        dy[base + v] = W::store(of);
      }
    }
    if (!DOT) continue;
    const float dw = wave_sum(part);  // the same value in every lane; 0 for a dropped copy
    if (lane == j) my_dw = dw;
  }
  if (!DOT) return;
  const float wl = lane < k ? w[t * k + lane] : 0.f;
  const float ssum = wave_sum(wl * my_dw);  // sum_i w_i dw_i
  if (lane < k) dl[t * k + lane] = wl * (my_dw - ssum);
}

// ---------------------------------------------------------------------------
// Gate gradients from the expert side, one wave per token. For a kept copy j,
// dh_j = w_j dout Wd is its hidden gradient and h_j its activation, so
// q_j = <dh_j, h_j> = w_j <dout, h_j Wd^T> = w_j dw_j; a dropped copy has
// q_j = 0. Then dl_j = w_j (dw_j - sum_i w_i dw_i) = q_j - w_j sum_i q_i.
// Each q_j is per-lane partials in word order, then a fixed butterfly.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void gate_grad_kernel(const uint4* __restrict__ dh, const uint4* __restrict__ h,
                                                        const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                        const int32_t* __restrict__ slot, int64_t T, int k, int64_t C,
                                                        int64_t VF, float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves only; no barriers below
  using W = Word<BF16>;
  float my_q = 0.f;  // lane j keeps q of copy j
  for (int j = 0; j < k; ++j) {
    const int sl = __builtin_amdgcn_readfirstlane(slot[t * k + j]);
    if (sl < 0) continue;  // q_j = 0
    const int64_t base = (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(idx[t * k + j])) * C + sl) * VF;
    float part = 0.f;
    for (int64_t v = lane; v < VF; v += 64) {
      float gf[W::N], hf[W::N];
      W::load(dh[base + v], gf);
      W::load(h[base + v], hf);
#pragma unroll
      for (int q = 0; q < W::N; ++q) part = fmaf(gf[q], hf[q], part);
    }
    const float q = wave_sum(part);
    if (lane == j) my_q = q;
  }
  const float wl = lane < k ? w[t * k + lane] : 0.f;
  const float qsum = wave_sum(my_q);  // lanes >= k hold 0
  if (lane < k) dl[t * k + lane] = my_q - wl * qsum;
}

// ---------------------------------------------------------------------------
// Dispatch backward, one wave per token: dx = dout + sum_j [kept] dX[e_j, s_j]
// + sum_j dl_j Wr[e_j], j ascending in each sum, fp32, rounded once.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void gather_dx_kernel(const uint4* __restrict__ dout, const uint4* __restrict__ dX,
                                                        const uint4* __restrict__ wr, const int32_t* __restrict__ idx,
                                                        const float* __restrict__ dl, const int32_t* __restrict__ slot,
                                                        int64_t T, int k, int64_t C, int64_t V, uint4* __restrict__ dx) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  using W = Word<BF16>;
  // U words per lane at a time; dout and the dX rows are read once
  // (non-temporal), the router rows are shared by many tokens (cached)
  constexpr int U = 4;
  for (int64_t v0 = 0; v0 < V; v0 += 64 * U) {
    float acc[U][W::N];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * 64 + lane;
      if (v < V) W::load(load_stream(dout + t * V + v), acc[u]);
    }
    for (int j = 0; j < k; ++j) {
      const int sl = __builtin_amdgcn_readfirstlane(slot[t * k + j]);
      if (sl < 0) continue;
      const int64_t e = __builtin_amdgcn_readfirstlane(idx[t * k + j]);
      uint4 g[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        if (v < V) g[u] = load_stream(dX + (e * C + sl) * V + v);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (v0 + u * 64 + lane < V) {
          float f[W::N];
          W::load(g[u], f);
#pragma unroll
          for (int q = 0; q < W::N; ++q) acc[u][q] += f[q];
        }
      }
    }
    for (int j = 0; j < k; ++j) {
      const int64_t e = __builtin_amdgcn_readfirstlane(idx[t * k + j]);
      const float c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(dl[t * k + j])));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        if (v < V) {
          float f[W::N];
          W::load(wr[e * V + v], f);
#pragma unroll
          for (int q = 0; q < W::N; ++q) acc[u][q] = fmaf(c, f[q], acc[u][q]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * 64 + lane;
      if (v < V) store_stream(dx + t * V + v, W::store(acc[u]));
    }
  }
}

// ---------------------------------------------------------------------------
// Router weight gradient: dWr[e][i] = sum_t sum_j [idx[t,j] = e] dl[t,j] x[t][i]
// and db[e] the same without x. Tokens are split into chunks (grid z): a
// block takes 16 experts x 256 columns of one chunk, accumulates in LDS (one
// column per thread, t then j ascending) and writes fp32 partials; a second
// kernel sums the chunks in order and rounds once. Deterministic.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void router_wgrad_part_kernel(const void* __restrict__ x,
                                                                const int32_t* __restrict__ idx,
                                                                const float* __restrict__ dl, int64_t T, int64_t tchunk,
                                                                int k, int E, int64_t d, float* __restrict__ part,
                                                                float* __restrict__ dbpart) {
  constexpr int EB = 16;
  __shared__ float acc[EB][256];
  __shared__ float dbs[EB];
  const int tid = threadIdx.x;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + tid;
  const int e0 = blockIdx.y * EB;
  const int64_t t0 = static_cast<int64_t>(blockIdx.z) * tchunk;
  const int64_t t1 = min(T, t0 + tchunk);
#pragma unroll
  for (int q = 0; q < EB; ++q) acc[q][tid] = 0.f;
  if (tid < EB) dbs[tid] = 0.f;
  __syncthreads();
  for (int64_t t = t0; t < t1; ++t) {
    for (int j = 0; j < k; ++j) {
      const int q = __builtin_amdgcn_readfirstlane(idx[t * k + j]) - e0;
      if (q < 0 || q >= EB) continue;  // uniform across the block
      const float c = dl[t * k + j];
      if (i < d) {
        const float xv = BF16 ? bf16_to_f32(static_cast<const bf16_t*>(x)[t * d + i])
                              : static_cast<const float*>(x)[t * d + i];
        acc[q][tid] = fmaf(c, xv, acc[q][tid]);
      }
      if (tid == 0 && blockIdx.x == 0) dbs[q] += c;
    }
  }
  __syncthreads();
  float* pz = part + static_cast<int64_t>(blockIdx.z) * E * d;
#pragma unroll
  for (int q = 0; q < EB; ++q) {
    const int e = e0 + q;
    if (e < E && i < d) pz[static_cast<int64_t>(e) * d + i] = acc[q][tid];
  }
  if (blockIdx.x == 0 && tid < EB && e0 + tid < E) dbpart[static_cast<int64_t>(blockIdx.z) * E + e0 + tid] = dbs[tid];
}

// The same with every expert in one block, for kWgradWideMinE <= E <=
// kWgradWideMaxE (with fewer experts the 16-expert blocks above waste little
// of their scan over the copies and keep more blocks in flight): a block
// takes 64 columns of one token chunk and holds acc[E][64] in LDS; wave w
// owns the experts e with e % 4 == w, so each accumulator has one writer,
// which adds in token order. A token's k copies are read once by lanes 0..k-1
// and broadcast; its 64 x values are read once per wave.
constexpr int kWgradWideMinE = 64, kWgradWideMaxE = 512;

template <bool BF16>
__global__ __launch_bounds__(256) void router_wgrad_wide_kernel(const void* __restrict__ x,
                                                                const int32_t* __restrict__ idx,
                                                                const float* __restrict__ dl, int64_t T, int64_t tchunk,
                                                                int k, int E, int64_t d, float* __restrict__ part,
                                                                float* __restrict__ dbpart) {
  extern __shared__ float wacc[];  // [E][64], then db [E]
  float* dbs = wacc + static_cast<int64_t>(E) * 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const int64_t t0 = static_cast<int64_t>(blockIdx.z) * tchunk;
  const int64_t t1 = min(T, t0 + tchunk);
  const bool want_db = blockIdx.x == 0;
  for (int q = tid; q < E * 64; q += 256) wacc[q] = 0.f;
  for (int q = tid; q < E; q += 256) dbs[q] = 0.f;
  __syncthreads();
  constexpr int U = 8;  // tokens whose loads are in flight together
  for (int64_t tb = t0; tb < t1; tb += U) {
    int e_l[U];
    float c_l[U], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = tb + u;
      const bool ok = t < t1;
      e_l[u] = ok && lane < k ? idx[t * k + lane] : 0;
      c_l[u] = ok && lane < k ? dl[t * k + lane] : 0.f;
      xv[u] = ok && i < d ? (BF16 ? bf16_to_f32(static_cast<const bf16_t*>(x)[t * d + i])
                                  : static_cast<const float*>(x)[t * d + i])
                          : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tb + u >= t1) break;
      for (int j = 0; j < k; ++j) {
        const int e = __builtin_amdgcn_readlane(e_l[u], j);
        if ((e & 3) != wave) continue;  // uniform across the wave
        const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c_l[u]), j));
        wacc[e * 64 + lane] = fmaf(c, xv[u], wacc[e * 64 + lane]);
        if (want_db && lane == 0) dbs[e] += c;
      }
    }
  }
  __syncthreads();
  float* pz = part + static_cast<int64_t>(blockIdx.z) * E * d;
  for (int e = wave; e < E; e += 4)
    if (i < d) pz[static_cast<int64_t>(e) * d + i] = wacc[e * 64 + lane];
  if (want_db)
    for (int e = tid; e < E; e += 256) dbpart[static_cast<int64_t>(blockIdx.z) * E + e] = dbs[e];
}

// Per expert, its routed copies in token order (lists from the slots pass):
// block (x, e, z) takes copies [cc z, cc z + cc) of expert e, 8 columns per
// lane (2048 per block, d % 8 == 0), and writes its fp32 partial sum of
// dl * x in copy order, plus (x == 0) the sum of dl, as partial row
// route_off[e] / cc + e + z. Those rows never overlap between experts (an
// expert with r copies has ceil(r / cc) chunks, at most one more than the
// whole chunks its copies span), so floor(T k / cc) + E + 1 rows suffice.
// Blocks past an expert's copies write nothing; the sum kernel reads only the
// chunks that exist.
__device__ inline int64_t wgrad_chunk_row(const int32_t* route_off, int e, int cc) {
  return static_cast<int64_t>(route_off[e]) / cc + e;
}

template <bool BF16>
__global__ __launch_bounds__(256) void router_wgrad_gather_kernel(
    const void* __restrict__ x, const int32_t* __restrict__ lcopy, const int32_t* __restrict__ ltok,
    const int32_t* __restrict__ route_off, const int32_t* __restrict__ routed, const float* __restrict__ dl,
    int cc, int64_t d, float* __restrict__ part, float* __restrict__ dbpart) {
  const int e = blockIdx.y, z = blockIdx.z;
  const int n = __builtin_amdgcn_readfirstlane(routed[e]);
  const int r0 = z * cc;
  if (r0 >= n) return;
  const int r1 = min(n, r0 + cc);
  const int64_t off = __builtin_amdgcn_readfirstlane(route_off[e]);
  const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  const bool live = c0 < d;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  float dbs = 0.f;
  // Copies whose loads are in flight together: every load of a batch is
  // issued without a branch, so the U row loads go out back to back instead
  // of one wait per copy. A whole batch reads U consecutive list entries; the
  // chunk's last, partial batch loads its last copy again in the places past
  // the end and leaves those out of the sums (a select, not a branch, so the
  // loads stay ahead of every use). A lane past the row's end loads column 0
  // and stores nothing.
  constexpr int U = 8;
  const int64_t cl = live ? c0 : 0;
  auto batch = [&](auto whole, int r) {
    constexpr bool W = decltype(whole)::value;
    float cf[U];
    uint4 xw[U][BF16 ? 1 : 2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = W ? r + u : min(r + u, r1 - 1);  // uniform
      const int ci = __builtin_amdgcn_readfirstlane(lcopy[off + rr]);
      const int64_t t = __builtin_amdgcn_readfirstlane(ltok[off + rr]);
      cf[u] = dl[ci];
      if constexpr (BF16) {
        xw[u][0] = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(x) + t * d + cl);
      } else {
        const uint4* px = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + t * d + cl);
        xw[u][0] = px[0];
        xw[u][1] = px[1];
      }
    }
    // in copy order
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xv[8];
      if constexpr (BF16) {
        const uint32_t ww[4] = {xw[u][0].x, xw[u][0].y, xw[u][0].z, xw[u][0].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xv[2 * q] = __uint_as_float(ww[q] << 16);
          xv[2 * q + 1] = __uint_as_float(ww[q] & 0xffff0000u);
        }
      } else {
        const uint32_t ww[8] = {xw[u][0].x, xw[u][0].y, xw[u][0].z, xw[u][0].w,
                                xw[u][1].x, xw[u][1].y, xw[u][1].z, xw[u][1].w};
#pragma unroll
        for (int q = 0; q < 8; ++q) xv[q] = __uint_as_float(ww[q]);
      }
      const bool in = W || r + u < r1;  // uniform
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float f = fmaf(cf[u], xv[q], acc[q]);
        acc[q] = in ? f : acc[q];
      }
      const float b = dbs + cf[u];
      dbs = in ? b : dbs;
    }
  };
  int r = r0;
  for (; r + U <= r1; r += U) batch(std::true_type{}, r);
  if (r < r1) batch(std::false_type{}, r);
  const int64_t row = wgrad_chunk_row(route_off, e, cc) + z;
  float* pz = part + row * d;
  if (live) {
    reinterpret_cast<float4*>(pz + c0)[0] = float4{acc[0], acc[1], acc[2], acc[3]};
    reinterpret_cast<float4*>(pz + c0)[1] = float4{acc[4], acc[5], acc[6], acc[7]};
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) dbpart[row] = dbs;
}

// Sums the chunk partials in chunk order: partial z of (e, i) at
// part[z][e][i] (nchunk chunks), or with routed (the gather layout, chunks of
// cc copies) at row route_off[e] / cc + e + z, ceil(routed[e] / cc) of them.
template <bool BF16>
__global__ __launch_bounds__(256) void router_wgrad_sum_kernel(const float* __restrict__ part,
                                                               const float* __restrict__ dbpart, int nchunk, int E,
                                                               int64_t d, void* __restrict__ dwr,
                                                               float* __restrict__ db,
                                                               const int32_t* __restrict__ routed,
                                                               const int32_t* __restrict__ route_off, int cc) {
  const int64_t n = static_cast<int64_t>(E) * d;
  // (first row, row stride, count) of the partials of expert e, in rows of d (or 1 for db)
  auto at = [&](int e, int64_t width, int64_t& first, int64_t& stride) {
    if (routed) {
      first = wgrad_chunk_row(route_off, e, cc) * width;
      stride = width;
      return (routed[e] + cc - 1) / cc;
    }
    first = static_cast<int64_t>(e) * width;
    stride = static_cast<int64_t>(E) * width;
    return nchunk;
  };
  // The chunks are added in chunk order; their loads go out eight at a time
  // (a hot expert has hundreds of chunks, and a chain of dependent load-adds
  // would wait out the memory latency once per chunk).
  auto chunk_sum = [&](const float* p, int64_t first, int64_t stride, int nz) {
    constexpr int G = 8;
    float s = 0.f;
    int z = 0;
    for (; z + G <= nz; z += G) {
      float v[G];
#pragma unroll
      for (int g = 0; g < G; ++g) v[g] = p[first + (z + g) * stride];
#pragma unroll
      for (int g = 0; g < G; ++g) s += v[g];
    }
    for (; z < nz; ++z) s += p[first + z * stride];
    return s;
  };
  for (int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; o < n;
       o += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int e = static_cast<int>(o / d);
    int64_t first, stride;
    const int nz = at(e, d, first, stride);
    const int64_t i = o - static_cast<int64_t>(e) * d;
    const float s = chunk_sum(part, first + i, stride, nz);
    if (BF16)
      static_cast<bf16_t*>(dwr)[o] = f32_to_bf16(s);
    else
      static_cast<float*>(dwr)[o] = s;
  }
  if (db && blockIdx.x == 0)
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      int64_t first, stride;
      const int nz = at(e, 1, first, stride);
      db[e] = chunk_sum(dbpart, first, stride, nz);
    }
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_transpose(const void* src, void* dst, int64_t batch, int64_t R, int64_t Cc, int64_t src_ld,
                            int64_t dst_ld, int64_t col_off, int64_t Rp, const int32_t* valid, int64_t src_bstride,
                            int64_t dst_bstride, bool bf16, hipStream_t s) {
  if (batch == 0 || Cc == 0 || Rp == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(ceil_div(Cc, 64)), static_cast<unsigned>(ceil_div(Rp, 64)),
                  static_cast<unsigned>(batch));
  const bool words = Cc % 8 == 0 && src_ld % 8 == 0 && dst_ld % 8 == 0 && col_off % 8 == 0 && Rp % 8 == 0 &&
                     src_bstride % 8 == 0 && dst_bstride % 8 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(dst) % 16 == 0;
  if (bf16 && words)
    transpose16_kernel<<<grid, dim3(256), 0, s>>>(static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), R,
                                                  Cc, src_ld, dst_ld, col_off, Rp, valid, src_bstride, dst_bstride);
  else if (bf16)
    transpose_kernel<uint16_t><<<grid, dim3(256), 0, s>>>(static_cast<const uint16_t*>(src),
                                                          static_cast<uint16_t*>(dst), R, Cc, src_ld, dst_ld,
                                                          col_off, Rp, valid, src_bstride, dst_bstride);
  else
    transpose_kernel<uint32_t><<<grid, dim3(256), 0, s>>>(static_cast<const uint32_t*>(src),
                                                          static_cast<uint32_t*>(dst), R, Cc, src_ld, dst_ld,
                                                          col_off, Rp, valid, src_bstride, dst_bstride);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const void* g, const void* u, void* h, const int32_t* kept, int E, int64_t C,
                             int64_t F, bool bf16, hipStream_t s) {
  if (E * C == 0) return hipSuccess;
  const int64_t VF = F * (bf16 ? 2 : 4) / 16;
  const dim3 grid(static_cast<unsigned>(E * C));
  if (bf16)
    swiglu_fwd_kernel<true><<<grid, dim3(256), 0, s>>>(static_cast<const uint4*>(g), static_cast<const uint4*>(u),
                                                       static_cast<uint4*>(h), kept, C, VF);
  else
    swiglu_fwd_kernel<false><<<grid, dim3(256), 0, s>>>(static_cast<const uint4*>(g), static_cast<const uint4*>(u),
                                                        static_cast<uint4*>(h), kept, C, VF);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* dh, const void* g, const void* u, void* dgu, const int32_t* kept, int E,
                             int64_t C, int64_t F, bool bf16, hipStream_t s) {
  if (E * C == 0) return hipSuccess;
  const int64_t VF = F * (bf16 ? 2 : 4) / 16;
  const dim3 grid(static_cast<unsigned>(E * C));
  const auto* a = static_cast<const uint4*>(dh);
  const auto* b = static_cast<const uint4*>(g);
  const auto* c = static_cast<const uint4*>(u);
  auto* o = static_cast<uint4*>(dgu);
  if (bf16)
    swiglu_bwd_kernel<true><<<grid, dim3(256), 0, s>>>(a, b, c, o, kept, C, VF);
  else
    swiglu_bwd_kernel<false><<<grid, dim3(256), 0, s>>>(a, b, c, o, kept, C, VF);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dout, const void* y, const int32_t* idx, const float* w,
                              const int32_t* slot, int64_t T, int64_t d, int k, int64_t C, bool bf16, void* dy,
                              float* dl, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k > 32) return hipErrorInvalidValue;
  const int64_t V = d * (bf16 ? 2 : 4) / 16;
  const dim3 grid(static_cast<unsigned>(ceil_div(T, 4)));
  const auto* a = static_cast<const uint4*>(dout);
  const auto* b = static_cast<const uint4*>(y);
  auto* o = static_cast<uint4*>(dy);
  if (bf16 && y)
    combine_bwd_kernel<true><<<grid, dim3(256), 0, s>>>(a, b, idx, w, slot, T, k, C, V, o, dl);
  else if (bf16)
    combine_bwd_kernel<true, false><<<grid, dim3(256), 0, s>>>(a, b, idx, w, slot, T, k, C, V, o, dl);
  else if (y)
    combine_bwd_kernel<false><<<grid, dim3(256), 0, s>>>(a, b, idx, w, slot, T, k, C, V, o, dl);
  else
    combine_bwd_kernel<false, false><<<grid, dim3(256), 0, s>>>(a, b, idx, w, slot, T, k, C, V, o, dl);
  return hipGetLastError();
}

hipError_t launch_gate_grad(const void* dh, const void* h, const int32_t* idx, const float* w, const int32_t* slot,
                            int64_t T, int64_t F, int k, int64_t C, bool bf16, float* dl, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k > 32) return hipErrorInvalidValue;
  const int64_t VF = F * (bf16 ? 2 : 4) / 16;
  const dim3 grid(static_cast<unsigned>(ceil_div(T, 4)));
  const auto* a = static_cast<const uint4*>(dh);
  const auto* b = static_cast<const uint4*>(h);
  if (bf16)
    gate_grad_kernel<true><<<grid, dim3(256), 0, s>>>(a, b, idx, w, slot, T, k, C, VF, dl);
  else
    gate_grad_kernel<false><<<grid, dim3(256), 0, s>>>(a, b, idx, w, slot, T, k, C, VF, dl);
  return hipGetLastError();
}

hipError_t launch_gather_dx(const void* dout, const void* dX, const void* wr, const int32_t* idx, const float* dl,
                            const int32_t* slot, int64_t T, int64_t d, int k, int64_t C, bool bf16, void* dx,
                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t V = d * (bf16 ? 2 : 4) / 16;
  const dim3 grid(static_cast<unsigned>(ceil_div(T, 4)));
  const auto* a = static_cast<const uint4*>(dout);
  const auto* b = static_cast<const uint4*>(dX);
  const auto* c = static_cast<const uint4*>(wr);
  auto* o = static_cast<uint4*>(dx);
  if (bf16)
    gather_dx_kernel<true><<<grid, dim3(256), 0, s>>>(a, b, c, idx, dl, slot, T, k, C, V, o);
  else
    gather_dx_kernel<false><<<grid, dim3(256), 0, s>>>(a, b, c, idx, dl, slot, T, k, C, V, o);
  return hipGetLastError();
}

namespace {
bool wgrad_gather(int E, int64_t d) { return E >= kWgradWideMinE && d % 8 == 0; }

// Copies per chunk of the gather kernel: a power of two in [64, 512] that
// makes about 1024 or more chunk blocks of 2048 columns.
int wgrad_copy_chunk(int64_t T, int k, int64_t d) {
  const int64_t want = T * k * ceil_div(d, 2048) / 1024;
  int cc = 64;
  while (cc < 512 && cc * 2 <= want) cc *= 2;
  return cc;
}
}  // namespace

size_t router_wgrad_scratch_floats(int64_t T, int k, int E, int64_t d) {
  if (wgrad_gather(E, d)) {
    const int64_t rows = T * k / wgrad_copy_chunk(T, k, d) + E + 1;
    return static_cast<size_t>(rows) * (d + 1);
  }
  return static_cast<size_t>(router_wgrad_chunks(T, E, d)) * E * (d + 1);
}

int router_wgrad_chunks(int64_t T, int E, int64_t d) {
  // wide kernel: about 2048 blocks of 64 columns; else about 8192 blocks of
  // 16 experts x 256 columns; chunks of at least 64 tokens
  const bool wide = E >= kWgradWideMinE && E <= kWgradWideMaxE;
  const int64_t tiles = wide ? ceil_div(d, 64) : ceil_div(d, 256) * ceil_div(E, 16);
  const int64_t by_work = ceil_div(wide ? 2048 : 8192, tiles);
  return static_cast<int>(std::max<int64_t>(1, std::min(by_work, ceil_div(T, 64))));
}

hipError_t launch_router_wgrad(const void* x, const int32_t* idx, const float* dl, int64_t T, int k, int E,
                               int64_t d, bool bf16, float* part, void* dwr, float* db, hipStream_t s,
                               const int32_t* routed, const int32_t* route_off, const int32_t* lcopy,
                               const int32_t* ltok) {
  const bool gather = wgrad_gather(E, d);
  if (gather && !(routed && route_off && lcopy && ltok)) return hipErrorInvalidValue;
  const int cc = gather ? wgrad_copy_chunk(T, k, d) : 0;
  // gather: chunk rows (T k / cc + E + 1) of d partials, then as many db partials
  const int nz = gather ? static_cast<int>(ceil_div(T, cc)) : router_wgrad_chunks(T, E, d);
  const int64_t tchunk = ceil_div(T, nz);
  float* dbpart = part + (gather ? (T * k / cc + E + 1) * d : static_cast<int64_t>(nz) * E * d);
  if (gather) {
    if (T > 0) {
      const dim3 grid(static_cast<unsigned>(ceil_div(d, 2048)), static_cast<unsigned>(E), static_cast<unsigned>(nz));
      if (bf16)
        router_wgrad_gather_kernel<true><<<grid, dim3(256), 0, s>>>(x, lcopy, ltok, route_off, routed, dl, cc, d,
                                                                    part, dbpart);
      else
        router_wgrad_gather_kernel<false><<<grid, dim3(256), 0, s>>>(x, lcopy, ltok, route_off, routed, dl, cc, d,
                                                                     part, dbpart);
    }
  } else if (E >= kWgradWideMinE && E <= kWgradWideMaxE) {
    const dim3 grid(static_cast<unsigned>(ceil_div(d, 64)), 1, static_cast<unsigned>(nz));
    const size_t lds = static_cast<size_t>(E) * 65 * sizeof(float);
    if (bf16)
      router_wgrad_wide_kernel<true><<<grid, dim3(256), lds, s>>>(x, idx, dl, T, tchunk, k, E, d, part, dbpart);
    else
      router_wgrad_wide_kernel<false><<<grid, dim3(256), lds, s>>>(x, idx, dl, T, tchunk, k, E, d, part, dbpart);
  } else {
    const dim3 grid(static_cast<unsigned>(ceil_div(d, 256)), static_cast<unsigned>(ceil_div(E, 16)),
                    static_cast<unsigned>(nz));
    if (bf16)
      router_wgrad_part_kernel<true><<<grid, dim3(256), 0, s>>>(x, idx, dl, T, tchunk, k, E, d, part, dbpart);
    else
      router_wgrad_part_kernel<false><<<grid, dim3(256), 0, s>>>(x, idx, dl, T, tchunk, k, E, d, part, dbpart);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned g2 = static_cast<unsigned>(std::min<int64_t>(ceil_div(static_cast<int64_t>(E) * d, 256), 4096));
  const int32_t* rt = gather ? routed : nullptr;
  if (bf16)
    router_wgrad_sum_kernel<true><<<dim3(g2), dim3(256), 0, s>>>(part, dbpart, nz, E, d, dwr, db, rt, route_off, cc);
  else
    router_wgrad_sum_kernel<false><<<dim3(g2), dim3(256), 0, s>>>(part, dbpart, nz, E, d, dwr, db, rt, route_off,
                                                                  cc);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  fill_i32_kernel<<<dim3(static_cast<unsigned>(std::min<int64_t>(ceil_div(n, 256), 1024))), dim3(256), 0, s>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace moe
