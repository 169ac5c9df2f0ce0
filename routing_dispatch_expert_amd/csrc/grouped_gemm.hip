// Experts of the MoE layer as a grouped GEMM over the fixed-capacity buckets
// (gfx950).
//
// Sources: "Expert Parallelism" (infra.bea.ai guide), section 1 - three
// weight matrices per expert; "Expert Parallelism & All-to-All"
// (neelmishra.github.io), "Tensor parallelism for experts" - gate, up and
// down projections; "Expert Parallelism" (klaylearn.com glossary) - local
// expert MLPs run as grouped GEMMs over the received buckets.
//
// For expert e and bucket row s < kept[e]:
//   h[e, s] = silu(X[e, s] Wg[e]^T) * (X[e, s] Wu[e]^T)     (GEMM 1, fused SwiGLU)
//   y[e, s] = h[e, s] Wd[e]^T                                (GEMM 2)
// Row tiles are listed per expert from kept[] on the device (mtile_off), so
// padding rows beyond kept[e] cost no tiles: a work-group maps its row-tile id
// to (expert, tile) by binary search over that prefix and exits when the id
// is past the last live tile.
#include "common.h"

namespace moe {
namespace {

// Find the expert owning row tile `mt`: largest e with mtile_off[e] <= mt.
__device__ inline int owner_expert(const int32_t* __restrict__ mtile_off, int E, int mt) {
  int lo = 0, hi = E;  // mtile_off[lo] <= mt < mtile_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mtile_off[mid] <= mt)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

__device__ inline float silu(float g) { return g / (1.0f + expf(-g)); }

// ---------------------------------------------------------------------------
// bf16 matrix-core GEMM: a 128 x 128 block of A B^T per work-group (4 waves,
// 2 x 2, each 64 x 64 as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16), K in steps
// of 64 through double-buffered LDS (rows padded by 8 elements). With SWIGLU,
// the 128 B rows are 64 gate rows then the same 64 up rows, and each wave
// holds gate and up accumulators of the same 32 output columns, so the SwiGLU
// product is taken in registers and only h is stored.
// Operand lane layout: lane l holds row (l % 32), K elements 8*(l/32) .. +8;
// accumulator element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, col l%32.
// ---------------------------------------------------------------------------
template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const bf16_t* __restrict__ A,
                                                        const bf16_t* __restrict__ B0,
                                                        const bf16_t* __restrict__ B1,
                                                        bf16_t* __restrict__ out,
                                                        const int32_t* __restrict__ kept,
                                                        const int32_t* __restrict__ mtile_off,
                                                        int E, int64_t C, int64_t K, int64_t N) {
  constexpr int BM = 128, BK = 64, LDK = BK + 8;
  constexpr int BNO = SWIGLU ? 64 : 128;  // output columns per work-group
  __shared__ bf16_t As[2][BM][LDK];
  __shared__ bf16_t Bs[2][128][LDK];

  const int mt = blockIdx.x;
  if (mt >= mtile_off[E]) return;
  const int e = owner_expert(mtile_off, E, mt);
  const int m0 = (mt - mtile_off[e]) * BM;
  const int rows = kept[e];
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BNO;

  const int tid = threadIdx.x;
  const bf16_t* Ae = A + static_cast<int64_t>(e) * C * K;
  const bf16_t* a_ptr[4];
  const bf16_t* b_ptr[4];
  int ld_row[4], ld_col[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = tid + 256 * r;
    ld_row[r] = c >> 3;
    ld_col[r] = (c & 7) * 8;
    const int64_t ar = min(m0 + ld_row[r], rows - 1);  // rows past kept: computed, never stored
    a_ptr[r] = Ae + ar * K + ld_col[r];
    const bf16_t* bsrc;
    int64_t br;
    if (SWIGLU) {
      bsrc = ld_row[r] < 64 ? B0 : B1;
      br = n0 + (ld_row[r] & 63);
    } else {
      bsrc = B0;
      br = n0 + ld_row[r];
    }
    br = min(br, N - 1);
    b_ptr[r] = bsrc + (static_cast<int64_t>(e) * N + br) * K + ld_col[r];
  }

  uint4 ra[4], rb[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool in = k0 + ld_col[r] < K;  // K is a multiple of 8
      ra[r] = in ? *reinterpret_cast<const uint4*>(a_ptr[r] + k0) : uint4{0, 0, 0, 0};
      rb[r] = in ? *reinterpret_cast<const uint4*>(b_ptr[r] + k0) : uint4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<uint4*>(&As[buf][ld_row[r]][ld_col[r]]) = ra[r];
      *reinterpret_cast<uint4*>(&Bs[buf][ld_row[r]][ld_col[r]]) = rb[r];
    }
  };

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int64_t nk = ceil_div(K, BK);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = static_cast<int>(kt & 1);
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[cur][wm * 64 + i * 32 + lr][ks * 16 + lk]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int brow = SWIGLU ? (j * 64 + wn * 32) : (wn * 64 + j * 32);
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][brow + lr][ks * 16 + lk]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  bf16_t* oute = out + static_cast<int64_t>(e) * C * N;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= rows) continue;
      if (SWIGLU) {
        const int64_t col = n0 + wn * 32 + lr;
        if (col < N) oute[row * N + col] = f32_to_bf16(silu(acc[i][0][r]) * acc[i][1][r]);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = n0 + wn * 64 + j * 32 + lr;
          if (col < N) oute[row * N + col] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 GEMM on the vector ALUs (fused multiply-add): 64 x 64 outputs per
// work-group, 4 x 4 per thread, K in steps of 16 through LDS. With SWIGLU the
// thread keeps gate and up sums of the same outputs.
// ---------------------------------------------------------------------------
template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B0,
                                                       const float* __restrict__ B1,
                                                       float* __restrict__ out,
                                                       const int32_t* __restrict__ kept,
                                                       const int32_t* __restrict__ mtile_off,
                                                       int E, int64_t C, int64_t K, int64_t N) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr int NB = SWIGLU ? 2 : 1;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[NB][BK][BN + 4];

  const int mt = blockIdx.x;
  if (mt >= mtile_off[E]) return;
  const int e = owner_expert(mtile_off, E, mt);
  const int m0 = (mt - mtile_off[e]) * BM;
  const int rows = kept[e];
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const float* Ae = A + static_cast<int64_t>(e) * C * K;
  const float* Bp[2] = {B0 + static_cast<int64_t>(e) * N * K,
                        SWIGLU ? B1 + static_cast<int64_t>(e) * N * K : nullptr};

  float acc[NB][4][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[b][i][j] = 0.f;

  for (int64_t k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + 256 * r;
      const int row = c >> 4, kk = c & 15;
      const bool in = k0 + kk < K;
      const int64_t ar = min(m0 + row, rows - 1);
      As[kk][row] = in ? Ae[ar * K + k0 + kk] : 0.f;
      const int64_t br = min(n0 + row, N - 1);
#pragma unroll
      for (int b = 0; b < NB; ++b) Bs[b][kk][row] = in ? Bp[b][br * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float bv = Bs[b][kk][tx * 4 + j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[b][i][j] = fmaf(a[i], bv, acc[b][i][j]);
        }
    }
    __syncthreads();
  }
  float* oute = out + static_cast<int64_t>(e) * C * N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + tx * 4 + j;
      if (col >= N) continue;
      oute[row * N + col] = SWIGLU ? silu(acc[0][i][j]) * acc[NB - 1][i][j] : acc[0][i][j];
    }
  }
}

}  // namespace

int grouped_gemm_bm(bool bf16, int64_t /*C*/) { return bf16 ? 128 : 64; }

hipError_t launch_gemm_gate_up(const void* buckets, const int32_t* kept, const int32_t* mtile_off,
                               const void* wg, const void* wu, int E, int64_t C, int64_t d,
                               int64_t d_ff, bool bf16, void* h, hipStream_t s) {
  const int bm = grouped_gemm_bm(bf16, C);
  const unsigned mtiles = static_cast<unsigned>(E * ceil_div(C, bm));  // upper bound of live tiles
  if (mtiles == 0) return hipSuccess;
  if (bf16)
    gemm_bf16_kernel<true><<<dim3(mtiles, static_cast<unsigned>(ceil_div(d_ff, 64))), dim3(256), 0, s>>>(
        static_cast<const bf16_t*>(buckets), static_cast<const bf16_t*>(wg), static_cast<const bf16_t*>(wu),
        static_cast<bf16_t*>(h), kept, mtile_off, E, C, d, d_ff);
  else
    gemm_f32_kernel<true><<<dim3(mtiles, static_cast<unsigned>(ceil_div(d_ff, 64))), dim3(256), 0, s>>>(
        static_cast<const float*>(buckets), static_cast<const float*>(wg), static_cast<const float*>(wu),
        static_cast<float*>(h), kept, mtile_off, E, C, d, d_ff);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const void* h, const int32_t* kept, const int32_t* mtile_off,
                            const void* wd, int E, int64_t C, int64_t d, int64_t d_ff, bool bf16,
                            void* y, hipStream_t s) {
  const int bm = grouped_gemm_bm(bf16, C);
  const unsigned mtiles = static_cast<unsigned>(E * ceil_div(C, bm));
  if (mtiles == 0) return hipSuccess;
  if (bf16)
    gemm_bf16_kernel<false><<<dim3(mtiles, static_cast<unsigned>(ceil_div(d, 128))), dim3(256), 0, s>>>(
        static_cast<const bf16_t*>(h), static_cast<const bf16_t*>(wd), nullptr, static_cast<bf16_t*>(y), kept,
        mtile_off, E, C, d_ff, d);
  else
    gemm_f32_kernel<false><<<dim3(mtiles, static_cast<unsigned>(ceil_div(d, 64))), dim3(256), 0, s>>>(
        static_cast<const float*>(h), static_cast<const float*>(wd), nullptr, static_cast<float*>(y), kept,
        mtile_off, E, C, d_ff, d);
  return hipGetLastError();
}

}  // namespace moe
