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
// The sum over j (ascending) is taken in fp32 with fused multiply-adds, added
// to x in fp32 and rounded once. A token with no kept copy is copied bit for
// bit (x + 0 would turn -0.0 into +0.0).
#include "common.h"

namespace moe {
namespace {

// One wave per token (WPT waves for short batches); lanes walk the row in
// 16-byte words (8 bf16 or 4 fp32 values), U words per lane at a time, read
// with the non-temporal hint (every word is read once). The
// token's copies are taken JB at a time: their slots, experts and gates are
// wave-uniform scalar loads, the words of every kept copy of the batch are in
// flight before any arithmetic, and the sum runs in ascending j.
template <bool BF16, int WPT, int U>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ x,
                                                      const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot, int64_t T, int k,
                                                      int64_t C, int64_t V, uint4* __restrict__ out) {
  constexpr int JB = 2;                  // copies whose words are in flight together
  constexpr int NE = BF16 ? 8 : 4;
  constexpr int LANES = 64 * WPT;        // threads sharing one token
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (4 / WPT) + threadIdx.x / LANES;
  if (t >= T) return;
  const int lane = threadIdx.x % LANES;
  const int32_t* st = slot + t * k;
  const int32_t* it = idx + t * k;
  const float* wt = w + t * k;
  bool any = false;
  for (int j = 0; j < k; ++j) any = any || st[j] >= 0;
  const uint4* xr = x + t * V;
  uint4* orow = out + t * V;
  for (int64_t v0 = lane; v0 < V; v0 += LANES * U) {
    uint4 xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + LANES * u;
      if (v < V) xv[u] = load_stream(&xr[v]);
    }
    if (!any) {  // every copy dropped: the row passes through bit for bit
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + LANES * u;
        if (v < V) store_stream(&orow[v], xv[u]);
      }
      continue;
    }
    float acc[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < NE; ++q) acc[u][q] = 0.f;
    for (int j0 = 0; j0 < k; j0 += JB) {
      int sl[JB];
      float wj[JB];
      const uint4* src[JB];
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const int j = j0 + jb;
        sl[jb] = j < k ? __builtin_amdgcn_readfirstlane(st[j]) : -1;
        wj[jb] = 0.f;
        src[jb] = y;
        if (sl[jb] >= 0) {
          wj[jb] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wt[j])));
          src[jb] = y + (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(it[j])) * C + sl[jb]) * V;
        }
      }
      uint4 yv[JB][U];
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        if (sl[jb] < 0) continue;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + LANES * u;
          if (v < V) yv[jb][u] = load_stream(&src[jb][v]);
        }
      }
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        if (sl[jb] < 0) continue;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t yw[4] = {yv[jb][u].x, yv[jb][u].y, yv[jb][u].z, yv[jb][u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (BF16) {
              acc[u][2 * q] = fmaf(wj[jb], __uint_as_float(yw[q] << 16), acc[u][2 * q]);
              acc[u][2 * q + 1] = fmaf(wj[jb], __uint_as_float(yw[q] & 0xffff0000u), acc[u][2 * q + 1]);
            } else {
              acc[u][q] = fmaf(wj[jb], __uint_as_float(yw[q]), acc[u][q]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + LANES * u;
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
                          const int32_t* slot, int64_t T, int64_t d, int k, int64_t C, bool bf16,
                          void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t V = d * (bf16 ? 2 : 4) / 16;
  const int wpt = row_waves_per_token(T);
  const dim3 grid(static_cast<unsigned>(ceil_div(T, 4 / wpt)));
  const auto* xv = static_cast<const uint4*>(x);
  const auto* yv = static_cast<const uint4*>(y);
  auto* ov = static_cast<uint4*>(out);
#define MOE_COMBINE(B, W) combine_kernel<B, W, 4><<<grid, dim3(256), 0, s>>>(xv, yv, idx, w, slot, T, k, C, V, ov)
  if (bf16 && wpt == 1 && V >= 768) {  // long rows (d >= 6144): 8 words per lane in flight
    combine_kernel<true, 1, 8><<<grid, dim3(256), 0, s>>>(xv, yv, idx, w, slot, T, k, C, V, ov);
  } else if (bf16) {
    if (wpt == 1) MOE_COMBINE(true, 1); else if (wpt == 2) MOE_COMBINE(true, 2); else MOE_COMBINE(true, 4);
  } else {
    if (wpt == 1) MOE_COMBINE(false, 1); else if (wpt == 2) MOE_COMBINE(false, 2); else MOE_COMBINE(false, 4);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
