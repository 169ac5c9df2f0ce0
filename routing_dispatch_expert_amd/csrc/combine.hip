// Combine of the MoE layer: the inverse permutation, gate-weighted and summed
// onto the residual (gfx950).
//
// Sources: "Expert Parallelism & All-to-All" (neelmishra.github.io), "All-to-all:
// the distributed transpose" - the combine exactly inverts the dispatch and a
// token's k expert outputs are weighted by their gates and added to the
// residual stream; "Expert Parallelism" (inferensys.com glossary), capacity
// entry - a dropped token passes through the layer unchanged.
//
// out[t] = x[t] + sum_j [slot[t,j] >= 0] w[t,j] * y[idx[t,j], slot[t,j]]
// A copy counts as kept only when 0 <= slot < C and 0 <= idx < E, so no
// index given by a caller reaches outside y. The sum over j (ascending) is
// taken in fp32 with fused multiply-adds, added to x in fp32 and rounded once. A token with no kept copy is copied bit for
// bit (x + 0 would turn -0.0 into +0.0).
#include "common.h"

namespace moe {
namespace {

// One 256-thread block per token; lanes walk the row in 16-byte words (8 bf16
// or 4 fp32 values), U words per lane, so a row of up to 256*U words takes one
// pass. Lane j of each wave loads copy j's slot, expert and gate (k <= 32), and
// the x words are requested in the same breath. A ballot over the slots gives
// the kept copies, which are walked in ascending j: the words of the next kept
// copy are in flight while the current one is accumulated. Every word is read
// and written once, with the non-temporal hint.
template <bool BF16, int U>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ x,
                                                      const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot, int64_t T, int k,
                                                      int E, int64_t C, int64_t V, uint4* __restrict__ out) {
  constexpr int NE = BF16 ? 8 : 4;
  const int64_t t = blockIdx.x;
  if (t >= T) return;
  const int lane = threadIdx.x;
  const int wl = threadIdx.x % 64;
  int s_l = -1, e_l = 0;
  float w_l = 0.f;
  if (wl < k) {
    s_l = slot[t * k + wl];
    e_l = idx[t * k + wl];
    w_l = w[t * k + wl];
  }
  const uint4* xr = x + t * V;
  uint4* orow = out + t * V;
  // taken while every lane is active: lanes past the row's end leave the loop below
  const uint64_t kept = __ballot(s_l >= 0 && s_l < C && e_l >= 0 && e_l < E);
  // row of kept copy j (a wave-uniform lane index) and its gate
  auto copy_row = [&](int j, float& wj) {
    const int e = __builtin_amdgcn_readlane(e_l, j);
    const int s = __builtin_amdgcn_readlane(s_l, j);
    wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), j));
    return y + (static_cast<int64_t>(e) * C + s) * V;
  };
  for (int64_t v0 = lane; v0 < V; v0 += 256 * U) {
    uint4 xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + 256 * u;
      if (v < V) xv[u] = load_stream(&xr[v]);
    }
    if (kept == 0) {  // every copy dropped: the row passes through bit for bit
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + 256 * u;
        if (v < V) store_stream(&orow[v], xv[u]);
      }
      continue;
    }
    float acc[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < NE; ++q) acc[u][q] = 0.f;
    uint64_t m = kept;
    float wc;
    const uint4* rc = copy_row(__builtin_ctzll(m), wc);
    m &= m - 1;
    uint4 cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + 256 * u;
      if (v < V) cur[u] = load_stream(&rc[v]);
    }
    while (true) {
      const bool more = m != 0;
      uint4 nxt[U];
      float wn = 0.f;
      if (more) {
        const uint4* rn = copy_row(__builtin_ctzll(m), wn);
        m &= m - 1;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + 256 * u;
          if (v < V) nxt[u] = load_stream(&rn[v]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t yw[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (BF16) {
            acc[u][2 * q] = fmaf(wc, __uint_as_float(yw[q] << 16), acc[u][2 * q]);
            acc[u][2 * q + 1] = fmaf(wc, __uint_as_float(yw[q] & 0xffff0000u), acc[u][2 * q + 1]);
          } else {
            acc[u][q] = fmaf(wc, __uint_as_float(yw[q]), acc[u][q]);
          }
        }
      }
      if (!more) break;
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
      wc = wn;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + 256 * u;
      if (v >= V) continue;
      const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
      uint32_t ow[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (BF16) {
          const float lo = __uint_as_float(xw[q] << 16) + acc[u][2 * q];
          const float hi = __uint_as_float(xw[q] & 0xffff0000u) + acc[u][2 * q + 1];
          ow[q] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
        } else {
          ow[q] = __float_as_uint(__uint_as_float(xw[q]) + acc[u][q]);
        }
      }
      store_stream(&orow[v], uint4{ow[0], ow[1], ow[2], ow[3]});
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* x, const void* y, const int32_t* idx, const float* w,
                          const int32_t* slot, int64_t T, int64_t d, int k, int E, int64_t C, bool bf16,
                          void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k > 32) return hipErrorInvalidValue;  // one lane per copy, k <= 32 lanes of a wave
  const int64_t V = d * (bf16 ? 2 : 4) / 16;
  const dim3 grid(static_cast<unsigned>(T));
  const auto* xv = static_cast<const uint4*>(x);
  const auto* yv = static_cast<const uint4*>(y);
  auto* ov = static_cast<uint4*>(out);
  // words per lane: the smallest of 1, 2, 4 that covers the row in one pass, else 8
  const int U = V <= 256 ? 1 : (V <= 512 ? 2 : (V <= 1024 ? 4 : 8));
#define MOE_COMBINE(B, UU) combine_kernel<B, UU><<<grid, dim3(256), 0, s>>>(xv, yv, idx, w, slot, T, k, E, C, V, ov)
#define MOE_COMBINE_U(B)                       \
  switch (U) {                                 \
    case 1: MOE_COMBINE(B, 1); break;          \
    case 2: MOE_COMBINE(B, 2); break;          \
    case 4: MOE_COMBINE(B, 4); break;          \
    default: MOE_COMBINE(B, 8); break;         \
  }
  if (bf16) {
    MOE_COMBINE_U(true);
  } else {
    MOE_COMBINE_U(false);
  }
#undef MOE_COMBINE_U
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
