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

// One work-group per token; threads walk the row in 16-byte words
// (8 bf16 or 4 fp32 values).
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ x,
                                                      const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot, int k,
                                                      int64_t C, int64_t V,
                                                      uint4* __restrict__ out) {
  __shared__ int64_t src[32];
  __shared__ float wt[32];
  __shared__ int nk;
  const int64_t t = blockIdx.x;
  if (threadIdx.x == 0) {
    int c = 0;
    for (int j = 0; j < k; ++j) {
      const int s = slot[t * k + j];
      if (s >= 0) {
        src[c] = (static_cast<int64_t>(idx[t * k + j]) * C + s) * V;
        wt[c] = w[t * k + j];
        ++c;
      }
    }
    nk = c;
  }
  __syncthreads();
  const int c = nk;
  const uint4* xr = x + t * V;
  uint4* orow = out + t * V;
  for (int64_t v = threadIdx.x; v < V; v += blockDim.x) {
    const uint4 xv = xr[v];
    if (c == 0) {
      orow[v] = xv;
      continue;
    }
    constexpr int NE = BF16 ? 8 : 4;
    float acc[NE];
#pragma unroll
    for (int q = 0; q < NE; ++q) acc[q] = 0.f;
    for (int j = 0; j < c; ++j) {
      const uint4 yv = y[src[j] + v];
      const float wj = wt[j];
      const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (BF16) {
          acc[2 * q] = fmaf(wj, __uint_as_float(yw[q] << 16), acc[2 * q]);
          acc[2 * q + 1] = fmaf(wj, __uint_as_float(yw[q] & 0xffff0000u), acc[2 * q + 1]);
        } else {
          acc[q] = fmaf(wj, __uint_as_float(yw[q]), acc[q]);
        }
      }
    }
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    uint32_t ow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (BF16) {
        const float lo = __uint_as_float(xw[q] << 16) + acc[2 * q];
        const float hi = __uint_as_float(xw[q] & 0xffff0000u) + acc[2 * q + 1];
        ow[q] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
      } else {
        ow[q] = __float_as_uint(__uint_as_float(xw[q]) + acc[q]);
      }
    }
    orow[v] = uint4{ow[0], ow[1], ow[2], ow[3]};
  }
}

}  // namespace

hipError_t launch_combine(const void* x, const void* y, const int32_t* idx, const float* w,
                          const int32_t* slot, int64_t T, int64_t d, int k, int64_t C, bool bf16,
                          void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t V = d * (bf16 ? 2 : 4) / 16;
  const dim3 grid(static_cast<unsigned>(T));
  const auto* xv = static_cast<const uint4*>(x);
  const auto* yv = static_cast<const uint4*>(y);
  auto* ov = static_cast<uint4*>(out);
  if (bf16)
    combine_kernel<true><<<grid, dim3(256), 0, s>>>(xv, yv, idx, w, slot, k, C, V, ov);
  else
    combine_kernel<false><<<grid, dim3(256), 0, s>>>(xv, yv, idx, w, slot, k, C, V, ov);
  return hipGetLastError();
}

}  // namespace moe
