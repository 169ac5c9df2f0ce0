// Internal declarations shared by the HIP kernels and the host library of the
// MoE-layer hot path (gfx950). Not part of the C ABI (see include/moe.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

using bf16_t = uint16_t;  // bfloat16 bit pattern

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tokens per tile of the expert histogram, its scan and the slot kernel.
constexpr int kTileTokens = 64;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }


__device__ inline float bf16_to_f32(bf16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN): one v_cvt_pk_bf16_f32.
__device__ inline bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// 16-byte store marked non-temporal: rows streamed out once (bucket scatter,
// combined output) skip the caches' allocate-and-keep path.
__device__ inline void store_stream(uint4* p, uint4 v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// A 16-byte load with the non-temporal hint (data read once, not to be kept
// in the caches).
__device__ inline uint4 load_stream(const uint4* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{w[0], w[1], w[2], w[3]};
}

// Block barrier for data exchanged through LDS only: it orders the block's
// LDS accesses across it, while global stores and loads still in flight stay
// in flight (no wait on the vector memory counter, unlike __syncthreads).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Ranks of one tile's copies, by one wave (64 lanes; LDS reads and writes of
// one wave stay in program order). ecp [ncp]: expert of each copy in
// flattened token order (-1: dropped); cnt [E]: zero on entry, the tile's
// histogram on exit. rank[i] (if given) = the number of copies before i in the
// tile with the same expert, -1 for a dropped copy. Copies are taken 64 at a
// time; lanes with the same expert form a group found by ballots over the
// expert-id bits, and a lane's rank within the round is the number of group
// lanes below it.
__device__ inline void rank_tile(const int* ecp, int ncp, int E, int* cnt, int32_t* rank) {
  const int lane = threadIdx.x & 63;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < ncp; c0 += 64) {
    const int i = c0 + lane;
    const int e = i < ncp ? ecp[i] : -1;
    const bool active = e >= 0;
    unsigned long long mask = __ballot(active);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (e >> bit) & 1;
      const unsigned long long m = __ballot(active && set);
      mask &= set ? m : ~m;
    }
    const int r = active ? cnt[e] + __popcll(mask & below) : -1;
    if (active && 63 - __clzll(mask) == lane) cnt[e] = r + 1;
    if (rank && i < ncp) rank[i] = r;
  }
}

// Ranks of one tile's copies by all the block's waves: wave w takes copies
// [64 w, 64 w + 64) (every wave of the block must call it). Within its 64
// copies a lane's rank is the number of lanes below it with the same expert
// (groups found by ballots over the expert-id bits) and the group's highest
// lane stores the group size as the chunk's count of that expert; after a
// barrier the counts become exclusive prefixes over the chunks, per expert,
// and a copy's rank is its rank in its chunk plus the count of its expert in
// the earlier chunks. Same result as rank_tile. cc: LDS scratch of
// ceil(ncp / 64) E ints (at most kRankChunkInts); cnt [E] gets the tile's
// histogram; ceil(ncp / 64) must not exceed the block's waves.
constexpr int kRankChunkInts = 8192;
// Whether a 1024-thread block over one 64-token tile ranks with all its waves.
__host__ __device__ inline bool tile_ranks_by_waves(int k, int E) { return k <= 16 && k * E <= kRankChunkInts; }
__device__ inline void rank_tile_waves(const int* ecp, int ncp, int E, int* cnt, int* cc, int32_t* rank) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = (ncp + 63) / 64;  // at most the block's waves: ncp <= 64 k, k <= 16
  for (int i = threadIdx.x; i < nch * E; i += blockDim.x) cc[i] = 0;
  lds_barrier();
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  int my_e = -1, my_r = 0;  // this lane's copy in chunk `wave` (nch <= 16 = waves of the block)
  if (wave < nch) {
    const int i = wave * 64 + lane;
    const int e = i < ncp ? ecp[i] : -1;
    const bool active = e >= 0;
    unsigned long long mask = __ballot(active);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (e >> bit) & 1;
      const unsigned long long m = __ballot(active && set);
      mask &= set ? m : ~m;
    }
    if (active) {
      my_e = e;
      my_r = __popcll(mask & below);
      if (63 - __clzll(mask) == lane) cc[wave * E + e] = __popcll(mask);
    }
  }
  lds_barrier();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < nch; ++w) {
      const int c = cc[w * E + e];
      cc[w * E + e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  lds_barrier();
  if (rank && wave < nch && wave * 64 + lane < ncp)
    rank[wave * 64 + lane] = my_e >= 0 ? my_r + cc[wave * E + my_e] : -1;
}

// ---- router (router.hip) ----
// Number of d-slices S the scores are split into (partials part[S][T][E]).
int router_splits(int64_t T, int64_t d, int E, bool bf16);
// Router scores as S partial slices part[S][T][E] over d (the route kernel
// adds them in slice order). With many experts they run on the grouped GEMM
// kernel.
hipError_t launch_router_logits(const void* x, const void* wr, int64_t T, int64_t d, int E, bool bf16,
                                int S, float* part, hipStream_t s);
// Sums the S partials (slice order) and the bias, writes logits_out if given,
// then top-k and gates; with tile_cnt, also the per-64-token-tile histogram
// (only when route_builds_histogram(k, E, T)). When route_rank_limited(P, M) the
// choice is limited to experts of the M best of P ranks (P <= 64, E % P == 0,
// M * E/P >= k); with S > 1 or a bias and no logits_out, the summed scores are
// then written over slice 0 of part.
bool route_builds_histogram(int k, int E, int64_t T);
bool route_rank_limited(int P, int M);
// With tile_cnt, also the ranks of each tile's copies (rank [T, k], optional;
// rank_tile). *zero = 0 when given (a counter the next kernel adds to).
hipError_t launch_route(const float* part, int S, const float* bias, int64_t T, int E, int k,
                        float* logits_out, int32_t* idx, float* w, int32_t* tile_cnt, int P, int M,
                        hipStream_t s, int32_t* rank = nullptr, int64_t* zero = nullptr);

// ---- permutation (permute.hip) ----
// With rank, also the ranks of each tile's copies (rank_tile); *zero = 0 when given.
hipError_t launch_tile_hist(const int32_t* idx, int64_t T, int k, int E, int32_t* tile_cnt,
                            hipStream_t s, int32_t* rank = nullptr, int64_t* zero = nullptr);
// Exclusive scan of the tile histogram over tiles, per expert; then counts,
// totals, send counts and (if mtile_off != nullptr) the GEMM row-tile prefix
// for row tiles of `bm` rows (and a second map for bm1 rows when mtile1 is
// given). 1 <= P <= E <= 4096. The scan block also zeroes clear[0 .. n_clear)
// (optional: the grouped GEMMs' split-K arrival counters).
// place [E] (optional): rank of each bucket for the send counts (default e / (E/P)).
hipError_t launch_scan(const int32_t* tile_cnt, int64_t nt, int E, int64_t C, int P,
                       int64_t row_bytes, int k, int64_t T, int32_t* tile_off, int32_t* routed,
                       int32_t* kept, int32_t* send, int64_t* totals, int bm, int32_t* mtile_off,
                       int32_t* src, hipStream_t s, const int32_t* place = nullptr, int bm1 = 0,
                       int32_t* mtile1 = nullptr, int32_t* clear = nullptr, int n_clear = 0);
// Slots from the scan and the in-tile ranks: slot [T, k] holds each copy's
// rank within its tile on entry (route or tile histogram) and its slot (-1:
// dropped) on exit; slot = tile_off + rank, kept below C. Also src (optional;
// kept rows only: the scan writes the padding) and totals[1] += tokens with no
// kept copy (optional; the scan zeroed it). Experts outside [0, E) are dropped.
hipError_t launch_slots_from_ranks(const int32_t* idx, int32_t* slot, const int32_t* tile_off, int64_t T, int k,
                                  int E, int64_t C, int32_t* src, int64_t* totals, hipStream_t s);
// The scan and the slots with the row scatter in one launch (block 0 scans
// while the others place and copy rows), when slot_scatter_fits(T, k, E):
// k <= 32, E <= 4096 and few enough earlier-tile counts to add up in each
// block (E (nt - 1) <= 65536, or k (nt - 1) <= 256 per token). Outputs as
// launch_scan followed by launch_slots_from_ranks and launch_scatter_rows;
// slot holds the ranks on entry; totals[1] must be zero on entry (zero it in
// the histogram launch).
bool slot_scatter_fits(int64_t T, int k, int E);
hipError_t launch_slot_scatter(const int32_t* tile_cnt, int E, int64_t C, int P, int64_t row_bytes, int k,
                               int64_t T, int32_t* tile_off, int32_t* routed, int32_t* kept, int32_t* send,
                               int64_t* totals, int bm, int32_t* mtile_off, int bm1, int32_t* mtile1,
                               int32_t* clear, int n_clear, const void* x, const int32_t* idx, int32_t* slot,
                               int32_t* src, void* buckets, hipStream_t s, const int32_t* place = nullptr);
// Replicated experts: instance offsets [E+1], expert [R] and rank [R] of each
// instance; then the instance of each copy from its rank among its expert's copies.
hipError_t launch_replica_layout(const int32_t* replicas, int E, int R, int P, int32_t* inst_off, int32_t* wmap,
                                 int32_t* place, hipStream_t s);
hipError_t launch_instances(const int32_t* idx, const int32_t* qrank, const int32_t* replicas,
                            const int32_t* inst_off, int64_t n, int R, int32_t* inst, hipStream_t s);
// Row-tile prefix of bm-row tiles over the counts kept[e] clamped to [0, C].
hipError_t launch_mtile_map(const int32_t* kept, int E, int64_t C, int bm, int32_t* mtile_off, hipStream_t s);
// With route_off ([E + 1], the exclusive scan of the routed counts), lcopy and
// ltok ([T * k]) list every routed copy per expert in token order: entry
// route_off[e] + r is copy r of expert e (flat index t * k + j, and t).
hipError_t launch_slots(const int32_t* idx, const int32_t* tile_off, int64_t T, int k, int E,
                        int64_t C, int32_t* slot, int32_t* src, int64_t* totals, hipStream_t s,
                        const int32_t* route_off = nullptr, int32_t* lcopy = nullptr, int32_t* ltok = nullptr);
// out[i] = sum of in[0 .. i) for i <= n (one work-group).
hipError_t launch_exclusive_scan(const int32_t* in, int n, int32_t* out, hipStream_t s);
hipError_t launch_scatter_rows(const void* x, const int32_t* idx, const int32_t* slot, int64_t T,
                               int k, int64_t C, int64_t row_bytes, void* buckets, hipStream_t s);

// ---- experts (grouped_gemm.hip) ----
// Row-tile height the grouped GEMM uses for these sizes (the mtile map must
// be built for the same value).
int grouped_gemm_bm(bool bf16, int64_t C);
// The same for GEMM 1 (gate/up, contraction length K = d) and GEMM 2 (down,
// K = d_ff) in the forward pass, and for the backward GEMMs that contract
// over d.
int grouped_gemm_bm_gate_up(bool bf16, int64_t C, int64_t K);
int grouped_gemm_bm_down(bool bf16, int64_t C, int64_t K);
int grouped_gemm_bm_contract_d(bool bf16, int64_t C, int64_t K);
// Scratch that lets the 256-column LDS-DMA GEMM split the tiles of its last,
// partly filled round over K: fp32 partial tiles (up to 320 x 256) of up to
// kSplitUnits work-groups and one arrival counter per split tile (cleared by
// the launcher).
constexpr int kSplitUnits = 256;
constexpr int kSplitTileElems = 320 * 256;
struct SplitK {
  float* part;    // [kSplitUnits][kSplitTileElems]
  int32_t* tick;  // [kSplitUnits]; each split tile's last block sets its counter back to zero
  bool zeroed = false;  // the counters are known to be zero (no clearing launch before the GEMM)
};
size_t split_k_bytes();
SplitK split_k_carve(void* base);  // base: 256-byte aligned, split_k_bytes() long
// GEMM 1: h = silu(X Wg^T) * (X Wu^T) on rows < kept. With wmap [E], bucket
// e uses the weights of expert wmap[e] (replicated experts). With sk, a last
// round that would leave most of the chip idle is split over K. With g and u
// (both or neither; only when gate_up_keeps_gu(bf16, C, d)) it also writes the
// rounded g = X Wg^T and u = X Wu^T, [E, C, d_ff], rows < kept.
bool gate_up_keeps_gu(bool bf16, int64_t C, int64_t d);
hipError_t launch_gemm_gate_up(const void* buckets, const int32_t* kept, const int32_t* mtile_off,
                               const void* wg, const void* wu, int E, int64_t C, int64_t d,
                               int64_t d_ff, bool bf16, void* h, hipStream_t s, const int32_t* wmap = nullptr,
                               const SplitK* sk = nullptr, void* g = nullptr, void* u = nullptr);
// GEMM 2: y = h Wd^T on rows < kept (wmap and sk as above). bm, if not 0,
// overrides the bf16 row-tile height (128 or 256; mtile_off built for it).
hipError_t launch_gemm_down(const void* h, const int32_t* kept, const int32_t* mtile_off,
                            const void* wd, int E, int64_t C, int64_t d, int64_t d_ff, bool bf16,
                            void* y, hipStream_t s, const int32_t* wmap = nullptr, const SplitK* sk = nullptr,
                            int bm = 0);

// out [slices][M][N] fp32: slice c = A [M][K] B [N][K]^T over the c-th of
// `slices` equal K ranges (whole 128-wide pairs of stages), bf16 operands, one
// group of 256-row tiles. Needs K % 128 == 0, N % 8 == 0 and
// 1 <= slices <= K / 128, else hipErrorInvalidValue.
hipError_t launch_gemm_rows_f32(const void* a, const void* b, int64_t M, int64_t K, int64_t N, int slices,
                                float* out, hipStream_t s);
// Weight gradients: out[e] [M][N] = A_e^T B_e over the kk[e] rows of group e,
// both operands K-major: A_e element (k, m) at a + e a_es + k lda + aoff + m,
// B_e element (k, n) at b + e b_es + k N + n. bf16; every group writes its
// whole M x N block (zero when kk[e] is 0). Needs M, N, lda and aoff
// multiples of 8 and aoff + M <= lda, else hipErrorInvalidValue.
hipError_t launch_gemm_tn(const void* a, int64_t lda, int64_t a_es, int64_t aoff, const void* b, int64_t b_es,
                          const int32_t* kk, int E, int64_t M, int64_t N, void* out, hipStream_t s);
// out = A [B0; B1] on rows < kept with B K-major: B0 [E][K0][N] holds K rows
// 0 .. K0 - 1 and B1 [E][K - K0][N] the rest (NULL when K0 == K). bf16,
// bm-row tiles, bm 256 or 320 (mtile_off built for bm); needs K % 128 == 0,
// K0 % 64 == 0 and N % 8 == 0, else hipErrorInvalidValue.
hipError_t launch_gemm_kmajor_b(const void* a, const int32_t* kept, const int32_t* mtile_off, const void* b0,
                                const void* b1, int64_t K0, int E, int64_t C, int64_t K, int64_t N, void* out,
                                hipStream_t s, const SplitK* sk = nullptr, int bm = 256);

// ---- backward (backward.hip) ----
// dst[b][c][col_off + r] = src[b][r][c] for r < valid[b] (or R), 0 for r < Rp.
hipError_t launch_transpose(const void* src, void* dst, int64_t batch, int64_t R, int64_t Cc, int64_t src_ld,
                            int64_t dst_ld, int64_t col_off, int64_t Rp, const int32_t* valid, int64_t src_bstride,
                            int64_t dst_bstride, bool bf16, hipStream_t s);
// h = silu(g) u on kept rows of [E][C][F].
hipError_t launch_swiglu_fwd(const void* g, const void* u, void* h, const int32_t* kept, int E, int64_t C,
                             int64_t F, bool bf16, hipStream_t s);
// dgu [E][C][2F] = [dh u silu'(g) | dh silu(g)] on kept rows.
hipError_t launch_swiglu_bwd(const void* dh, const void* g, const void* u, void* dgu, const int32_t* kept, int E,
                             int64_t C, int64_t F, bool bf16, hipStream_t s);
// dy rows of kept copies = w dout; with y (the expert outputs) also dl [T][k],
// the gate gradients (y NULL: dl untouched).
hipError_t launch_combine_bwd(const void* dout, const void* y, const int32_t* idx, const float* w,
                              const int32_t* slot, int64_t T, int64_t d, int k, int64_t C, bool bf16, void* dy,
                              float* dl, hipStream_t s);
// dl [T][k], the gate gradients, from the hidden gradients dh = dy Wd and
// activations h of the kept copies ([E][C][F] each).
hipError_t launch_gate_grad(const void* dh, const void* h, const int32_t* idx, const float* w, const int32_t* slot,
                            int64_t T, int64_t F, int k, int64_t C, bool bf16, float* dl, hipStream_t s);
// dx = dout + sum_j [kept] dX[e_j, s_j] + sum_j dl_j Wr[e_j].
hipError_t launch_gather_dx(const void* dout, const void* dX, const void* wr, const int32_t* idx, const float* dl,
                            const int32_t* slot, int64_t T, int64_t d, int k, int64_t C, bool bf16, void* dx,
                            hipStream_t s);
// dWr [E][d] (dtype) and db [E] fp32 (may be NULL) from dl and x; part is fp32
// scratch of router_wgrad_scratch_floats() floats. With the routed-copy
// lists of launch_slots (route_off, lcopy, ltok, routed counts), 64 or more
// experts and d % 8 == 0, each expert gathers its own copies' rows instead.
int router_wgrad_chunks(int64_t T, int E, int64_t d);
size_t router_wgrad_scratch_floats(int64_t T, int k, int E, int64_t d);
hipError_t launch_router_wgrad(const void* x, const int32_t* idx, const float* dl, int64_t T, int k, int E,
                               int64_t d, bool bf16, float* part, void* dwr, float* db, hipStream_t s,
                               const int32_t* routed = nullptr, const int32_t* route_off = nullptr,
                               const int32_t* lcopy = nullptr, const int32_t* ltok = nullptr);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// ---- combine (combine.hip) ----
// A copy is kept when 0 <= slot < C and 0 <= idx < E (E buckets in y).
hipError_t launch_combine(const void* x, const void* y, const int32_t* idx, const float* w,
                          const int32_t* slot, int64_t T, int64_t d, int k, int E, int64_t C, bool bf16,
                          void* out, hipStream_t s);

}  // namespace moe
