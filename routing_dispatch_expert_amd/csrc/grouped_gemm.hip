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
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

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

// Rows of bucket e that hold data: kept[e] clamped to [0, C], so a count
// beyond the capacity never reaches past the bucket.
__device__ inline int bucket_rows(const int32_t* __restrict__ kept, int e, int64_t C) {
  return static_cast<int>(min(max(static_cast<int64_t>(kept[e]), int64_t{0}), C));
}

__device__ inline float silu(float g) { return g / (1.0f + expf(-g)); }

// silu for results rounded to bf16 next: hardware 2^x and reciprocal (each
// within about 1 ulp of fp32), far below the 2^-9 of the bf16 rounding.
__device__ inline float silu_bf16(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

// ---------------------------------------------------------------------------
// bf16 matrix-core GEMM, one BM x BN block of A B^T per work-group of 4 waves
// (2 x 2). Each wave owns a (BM/2) x (BN/2) block as TM x TN tiles of
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators. K advances 64 at a time
// through two LDS buffers: the next step's tile is fetched into registers
// while the current one feeds the matrix cores, so one barrier per step.
// LDS rows are 64 elements (eight 16-byte chunks) with chunk c of row r kept
// at position c ^ (r % 8), so the 32 rows a wave reads at once spread over
// all banks.
// With SWIGLU the BN rows of B are BN/2 gate rows then the same BN/2 up rows,
// and each wave holds gate and up accumulators of the same output columns, so
// silu(g) * u is taken in registers and only h is stored.
// Operand lane layout: lane l holds row (l % 32), K elements 8*(l/32) .. +8;
// accumulator element q of lane l is row 8*(q/4) + 4*(l/32) + q%4, col l%32.
// Tile order: the live tiles (kept rows only) are numbered expert by expert;
// inside an expert, column tiles come in groups of kGroupN, and each group
// walks all of the expert's row tiles. Hardware hands block b to XCD b % 8;
// block b takes tile (b % 8) * ceil(L / 8) + b / 8 of the L live tiles, so
// each XCD works through one contiguous eighth, and the blocks running
// together on an XCD share the expert's row tiles (A) and a group of weight
// tiles (B) in its L2.
// ---------------------------------------------------------------------------
constexpr int kGroupN = 8;
// Weight-gradient launches (K-major A and B) keep one resident block per CU
// that walks its XCD's tiles in turn.
constexpr bool kPersistAt = true;

// Expert, first row and column tile of live tile `lid`. Without a row-tile
// map every one of the E groups has ceil(C / BM) row tiles. With the kept
// counts (and the map) an expert's kept rows are shared evenly by its row
// tiles, in whole 32-row blocks: S = 32 ceil(kept / (32 n)) rows each for n =
// ceil(kept / BM) tiles, so no tile is left nearly empty (1024 rows: four of
// 256, not 320, 320, 320 and 64); *r1_out is then the tile's row end.
template <int BM>
__device__ inline void tile_coords(const int32_t* __restrict__ mtile_off, int E, int nt_count, int64_t lid,
                                   int* e_out, int* m0_out, int* nt_out, int64_t C = 0,
                                   const int32_t* __restrict__ kept = nullptr, int* r1_out = nullptr) {
  const int mt_all = static_cast<int>((C + BM - 1) / BM);
  // Without a row-tile map every group has the same tiles (the weight
  // gradients, where a tile's cost follows its group's rows of K): the groups
  // are dealt to the 8 XCDs in turn, so XCD x (which takes a contiguous eighth
  // of the tile ids) holds groups x, x + 8, x + 16, ... rather than a run of
  // neighbours, and a run of heavy experts is spread over all of them.
  const int eg = mtile_off ? owner_expert(mtile_off, E, static_cast<int>(lid / nt_count))
                           : static_cast<int>(lid / (static_cast<int64_t>(mt_all) * nt_count));
  const int e = (mtile_off || E % 8) ? eg : (eg % (E / 8)) * 8 + eg / (E / 8);
  const int mte = mtile_off ? mtile_off[e + 1] - mtile_off[e] : mt_all;
  const int64_t li = lid - (mtile_off ? static_cast<int64_t>(mtile_off[e]) * nt_count
                                      : static_cast<int64_t>(eg) * mt_all * nt_count);
  const int64_t grp = li / (static_cast<int64_t>(mte) * kGroupN);
  const int r = static_cast<int>(li - grp * mte * kGroupN);
  *e_out = e;
  *nt_out = static_cast<int>(grp * kGroupN + r / mte);
  if (kept && mtile_off) {
    const int n = bucket_rows(kept, e, C);
    const int S = 32 * ((n + 32 * mte - 1) / (32 * mte));  // <= BM, as mte = ceil(n / BM)
    *m0_out = (r % mte) * S;
    *r1_out = min(n, *m0_out + S);
  } else {
    *m0_out = (r % mte) * BM;
    if (r1_out) *r1_out = INT_MAX;
  }
}

// Live tile of block b when the first n live tiles are spread over the XCDs
// (block b runs on XCD b % 8 and takes tile (b % 8) * ceil(n / 8) + b / 8).
__device__ inline int64_t xcd_tile(int64_t b, int64_t n) {
  const int64_t per_xcd = (n + 7) / 8;
  const int64_t slot = b / 8;
  if (slot >= per_xcd) return -1;
  const int64_t lid = (b % 8) * per_xcd + slot;
  return lid < n ? lid : -1;
}

template <int BM>
__device__ inline bool tile_of_block(const int32_t* __restrict__ mtile_off, int E, int nt_count,
                                     int* e_out, int* m0_out, int* nt_out) {
  const int64_t lid = xcd_tile(blockIdx.x, static_cast<int64_t>(mtile_off[E]) * nt_count);
  if (lid < 0) return false;
  tile_coords<BM>(mtile_off, E, nt_count, lid, e_out, m0_out, nt_out);
  return true;
}

// Split-K of the last round. With G work-groups resident at once and L live
// tiles, rem = L % G tiles would run alone in a last round. When G / rem >= 2
// each of them is cut into s = min(G / rem, nk / 2, kMaxSplit) K ranges of
// whole stage pairs, one block each (rem * s <= G blocks), after the blocks of
// the L - rem whole tiles. Block b then holds K stages [kb, ke) of split tile
// ti as its chunk c of s; s = 1 means a whole tile.
constexpr int kMaxSplit = 8;

struct Work {
  int e, m0, nt;
  int r1;  // the tile's row end (INT_MAX: the group's)
  int64_t kb, ke;
  int s, c, ti;
};

// With slices > 1 instead (and G = 0), block b takes K range b % slices of
// live tile b / slices, and the caller keeps the slices' results apart.
template <int BM>
__device__ inline bool work_of_block(const int32_t* __restrict__ mtile_off, int E, int nt_count, int64_t nk,
                                     int G, Work* w, int64_t C = 0, int slices = 1, int64_t bid = -1,
                                     const int32_t* __restrict__ kept = nullptr) {
  if (bid < 0) bid = blockIdx.x;
  const int64_t live = (mtile_off ? static_cast<int64_t>(mtile_off[E]) : E * ((C + BM - 1) / BM)) * nt_count;
  if (slices > 1) {
    const int64_t lid = bid / slices;
    if (lid >= live) return false;
    w->s = 1;
    w->ti = 0;
    w->c = static_cast<int>(bid % slices);
    const int64_t pairs = nk / 2;
    w->kb = 2 * (w->c * pairs / slices);
    w->ke = 2 * ((w->c + 1) * pairs / slices);
    tile_coords<BM>(mtile_off, E, nt_count, lid, &w->e, &w->m0, &w->nt, C, kept, &w->r1);
    return true;
  }
  int64_t rem = G > 0 ? live % G : 0;
  int64_t s = rem > 0 ? G / rem : 1;
  s = s < nk / 2 ? s : nk / 2;
  s = s < kMaxSplit ? s : kMaxSplit;
  if (s < 2) rem = 0, s = 1;
  const int64_t whole = live - rem;
  // xcd_tile hands the whole tiles to the first ceil(whole / 8) * 8 blocks
  // (some of them idle); the split blocks come after those
  const int64_t whole_blocks = (whole + 7) / 8 * 8;
  int64_t lid;
  w->s = 1;
  w->c = 0;
  w->ti = 0;
  w->kb = 0;
  w->ke = nk;
  if (bid < whole_blocks) {
    lid = xcd_tile(bid, whole);
    if (lid < 0) return false;
  } else {
    const int64_t u = bid - whole_blocks;
    if (u >= rem * s) return false;
    w->s = static_cast<int>(s);
    w->ti = static_cast<int>(u / s);
    w->c = static_cast<int>(u % s);
    lid = whole + w->ti;
    const int64_t pairs = nk / 2;
    w->kb = 2 * (w->c * pairs / s);
    w->ke = 2 * ((w->c + 1) * pairs / s);
  }
  tile_coords<BM>(mtile_off, E, nt_count, lid, &w->e, &w->m0, &w->nt, C, kept, &w->r1);
  return true;
}

// Raw buffer resource over [base, base + bytes): loads past `bytes` return 0.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

__device__ inline uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0);
  return uint4{static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), static_cast<uint32_t>(v[2]),
               static_cast<uint32_t>(v[3])};
}

// Scheduling hints: instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;

// One k-step's schedule: NR groups, each one LDS read and its share of the NM
// matrix instructions (shares differ by at most one), the read first or last.
template <int C, bool READS_FIRST>
__device__ inline void interleave_group() {
  if constexpr (READS_FIRST) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  if constexpr (C > 0) __builtin_amdgcn_sched_group_barrier(kSchedMfma, C, 0);
  if constexpr (!READS_FIRST) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
}

template <int NM, int NR, bool READS_FIRST, int... G>
__device__ inline void interleave_groups(std::integer_sequence<int, G...>) {
  (interleave_group<(NM * (G + 1)) / NR - (NM * G) / NR, READS_FIRST>(), ...);
}


// Epilogue of one wave's (32 TM) x (32 TN) accumulator block (v_mfma 32x32
// layout: element q of lane l is row 8 (q / 4) + 4 (l / 32) + q % 4, column
// l % 32 of its tile), staged through CAP bytes of LDS that no other wave
// touches: the results are rounded to bf16 into rows padded by 16 bytes (or,
// without PAD, swizzled) so the two half-waves, four rows apart, write
// different banks; then whole 16-byte row chunks are stored, so every global
// store is coalesced. With
// SWIGLU the tiles j < TN/2 hold gate and j + TN/2 the matching up values, and
// silu(gate) * up is stored. Rows >= rows and columns >= N are not written
// (N % 8 == 0). NT marks the stores non-temporal (results nothing reads soon).
constexpr int staged_rows(int wr, int rs, int cap) {
  for (int h = wr; h >= 32; h -= 32)
    if (wr % h == 0 && h * rs <= cap) return h;
  return 0;
}

template <int TM, int TN, bool SWIGLU, int CAP, bool PAD = true, bool NT = false>
__device__ inline void store_wave_tile(const f32x16 (&acc)[TM][TN], char* eb, bf16_t* __restrict__ out,
                                       int row0, int rows, int64_t col0, int64_t N, int lane) {
  constexpr int WR = TM * 32;                        // rows of the wave's block
  constexpr int OC = SWIGLU ? TN * 16 : TN * 32;     // output columns of the wave's block
  constexpr int RS = OC * 2 + (PAD ? 16 : 0);        // LDS row stride, bytes
  // without padding, rows with bit 2 of the row index set keep their 64-byte
  // halves swapped, which separates the half-waves just as well
  auto at = [&](int r, int byte) { return r * RS + (PAD ? byte : (byte ^ (((r >> 2) & 1) << 6))); };
  constexpr int HR = staged_rows(WR, RS, CAP);       // rows staged per pass
  constexpr int CPR = OC / 8;                        // 16-byte chunks per row
  static_assert(HR > 0 && HR * RS <= CAP, "staging rows fit the LDS slice");
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int pass = 0; pass < WR / HR; ++pass) {
#pragma unroll
    for (int ii = 0; ii < HR / 32; ++ii) {
      const int i = pass * (HR / 32) + ii;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = ii * 32 + 8 * (q >> 2) + 4 * lk + (q & 3);
#pragma unroll
        for (int j = 0; j < OC / 32; ++j) {
          const float v = SWIGLU ? silu_bf16(acc[i][j][q]) * acc[i][j + TN / 2][q] : acc[i][j][q];
          *reinterpret_cast<bf16_t*>(eb + at(r, (j * 32 + lr) * 2)) = f32_to_bf16(v);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0): rows staged
#pragma unroll
    for (int c = lane; c < HR * CPR; c += 64) {
      const int r = c / CPR, ch = c % CPR;
      const int grow = row0 + pass * HR + r;
      const int64_t gcol = col0 + ch * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(eb + at(r, ch * 16));
      if (grow < rows && gcol < N) {
        if (NT)
          store_stream(reinterpret_cast<uint4*>(out + grow * N + gcol), v);
        else
          *reinterpret_cast<uint4*>(out + grow * N + gcol) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // reads done before reuse
  }
}

template <int BM, int BN, bool SWIGLU>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, BM >= 256 ? 1 : 2))) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
    bf16_t* __restrict__ out, const int32_t* __restrict__ kept, const int32_t* __restrict__ mtile_off,
    int E, int64_t C, int64_t K, int64_t N, int nt_count, const int32_t* __restrict__ wmap) {
  constexpr int BK = 64;
  constexpr int TM = BM / 64, TN = BN / 64;      // 32 x 32 tiles per wave
  constexpr int AL = BM * (BK / 8) / 256;        // 16-byte chunks per thread
  constexpr int BL = BN * (BK / 8) / 256;
  constexpr int BNO = SWIGLU ? BN / 2 : BN;      // output columns per work-group
  constexpr int NMFMA = TM * TN;                 // MFMAs per 16-wide K step
  constexpr int NFRAG = TM + TN;                 // LDS fragment reads per K step
  __shared__ uint4 As[2][BM * 8];
  __shared__ uint4 Bs[2][BN * 8];

  int e, m0, nt;
  if (!tile_of_block<BM>(mtile_off, E, nt_count, &e, &m0, &nt)) return;
  // the tile is the same for the whole work-group: keep it in scalar registers
  e = __builtin_amdgcn_readfirstlane(e);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  nt = __builtin_amdgcn_readfirstlane(nt);
  const int rows = __builtin_amdgcn_readfirstlane(bucket_rows(kept, e, C));
  const int64_t n0 = static_cast<int64_t>(nt) * BNO;

  // Global operands through raw buffer loads: one 32-bit offset per chunk,
  // the K position in a scalar offset. Rows past C (A) or N (B) and K past
  // the end read as zero; rows in [kept, C) are padding whose results are
  // never stored.
  const int tid = threadIdx.x;
  const int lrow = tid >> 3;   // first row this thread loads; then every 32nd
  const int lch = tid & 7;     // 16-byte chunk within the 64-element row
  const uint32_t a_bytes = static_cast<uint32_t>(C * K * 2);
  const uint32_t b_bytes = static_cast<uint32_t>(N * K * 2);
  const auto ra_src = buffer_rsrc(A + static_cast<int64_t>(e) * C * K, a_bytes);
  const int we = wmap ? __builtin_amdgcn_readfirstlane(wmap[e]) : e;  // expert whose weights this row tile uses
  const auto rb_src0 = buffer_rsrc(B0 + static_cast<int64_t>(we) * N * K, b_bytes);
  const auto rb_src1 = buffer_rsrc((SWIGLU ? B1 : B0) + static_cast<int64_t>(we) * N * K, b_bytes);
  uint32_t a_off[AL], b_off[BL];
#pragma unroll
  for (int r = 0; r < AL; ++r) a_off[r] = static_cast<uint32_t>((m0 + lrow + 32 * r) * K * 2 + lch * 16);
#pragma unroll
  for (int r = 0; r < BL; ++r) {
    const int br = lrow + 32 * r;
    const int64_t bn = n0 + (SWIGLU ? (br % (BN / 2)) : br);
    b_off[r] = bn < N ? static_cast<uint32_t>(bn * K * 2 + lch * 16) : 0x80000000u;
  }
  uint4 ra[AL], rb[BL];
  auto gload = [&](int64_t k0) {
    const uint32_t mask = (k0 + lch * 8 < K) ? 0u : 0x80000000u;  // K is a multiple of 8
    const uint32_t soff = static_cast<uint32_t>(k0 * 2);
#pragma unroll
    for (int r = 0; r < AL; ++r) ra[r] = buffer_load16(ra_src, a_off[r] | mask, soff);
#pragma unroll
    for (int r = 0; r < BL; ++r)
      rb[r] = buffer_load16((SWIGLU && r >= BL / 2) ? rb_src1 : rb_src0, b_off[r] | mask, soff);
  };
  // LDS rows are eight 16-byte chunks; chunk c of row r sits at c ^ ((r / 2) % 8)
  // so 16 lanes reading 16 consecutive rows hit 16 distinct bank groups.
  const int swz = lch ^ ((lrow >> 1) & 7);  // rows lrow + 32 r share (row / 2) % 8
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < AL; ++r) As[buf][(lrow + 32 * r) * 8 + swz] = ra[r];
#pragma unroll
    for (int r = 0; r < BL; ++r) Bs[buf][(lrow + 32 * r) * 8 + swz] = rb[r];
  };

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
  int a_row[TM], b_row[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row[i] = (wm * (BM / 2) + i * 32 + lr) * 8;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int br;
    if (SWIGLU)
      br = (j < TN / 2) ? (wn * (BN / 4) + j * 32) : (BN / 2 + wn * (BN / 4) + (j - TN / 2) * 32);
    else
      br = wn * (BN / 2) + j * 32;
    b_row[j] = (br + lr) * 8;
  }
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // Fragments of one 16-wide K step, double-buffered in registers so the
  // next step's LDS reads are in flight while this step's MFMAs issue.
  bf16x8 fa[2][TM], fb[2][TN];
  const int rsw = (lr >> 1) & 7;  // (row / 2) % 8 of every row this lane reads
  auto fload = [&](int buf, int ks, int slot) {
    const int pc = (ks * 2 + lk) ^ rsw;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[slot][i] = *reinterpret_cast<const bf16x8*>(&As[buf][a_row[i] + pc]);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[slot][j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][b_row[j] + pc]);
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
  };

  // Per 64-wide K stage kt (LDS buffer cur holds it; the fragments of its
  // first 16-wide step are in slot 0; the registers ra/rb hold stage kt + 1,
  // fetched one stage earlier):
  //   step 0: read step 1's fragments
  //   step 1: read step 2's fragments
  //   step 2: read step 3's fragments; store stage kt + 1 into the other LDS
  //           buffer, then fetch stage kt + 2 into ra/rb
  //   barrier; read stage kt + 1's step 0 fragments
  //   step 3: MFMAs only (they overlap the barrier and those reads)
  // A fetch thus has a whole stage of MFMAs to arrive.
  const int64_t nk = ceil_div(K, BK);
  auto stage = [&](int64_t kt, bool store_next, bool fetch) {
    const int cur = static_cast<int>(kt & 1);
    fload(cur, 1, 1);
    mfmas(0);
#pragma unroll
    for (int g = 0; g < NFRAG; ++g) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMFMA / NFRAG, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    fload(cur, 2, 0);
    mfmas(1);
#pragma unroll
    for (int g = 0; g < NFRAG; ++g) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMFMA / NFRAG, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    fload(cur, 3, 1);
    if (store_next) sstore(cur ^ 1);
    if (fetch) gload((kt + 2) * BK);
    mfmas(0);
    if (store_next && fetch) {
#pragma unroll
      for (int g = 0; g < NFRAG; ++g) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMFMA / NFRAG, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, (AL + BL) / NFRAG, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, (AL + BL) / NFRAG, 0);
      }
    }
    if (store_next) {
      __builtin_amdgcn_sched_barrier(0);  // nothing moves across the barrier
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      fload(cur ^ 1, 0, 0);
    }
    mfmas(1);
#pragma unroll
    for (int g = 0; g < NFRAG; ++g) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMFMA / NFRAG, 0);
    }
  };

  gload(0);
  sstore(0);
  if (nk > 1) gload(BK);
  __syncthreads();
  fload(0, 0, 0);
  int64_t kt = 0;
  for (; kt + 2 < nk; ++kt) stage(kt, true, true);  // no branches inside a stage
  if (kt + 1 < nk) stage(kt++, true, false);
  stage(kt, false, false);

  // the stage buffers are free: one per wave for the epilogue
  __syncthreads();
  char* eb = reinterpret_cast<char*>(wave == 0 ? As[0] : wave == 1 ? As[1] : wave == 2 ? Bs[0] : Bs[1]);
  store_wave_tile<TM, TN, SWIGLU, (BM < BN ? BM : BN) * 8 * 16>(
      acc, eb, out + static_cast<int64_t>(e) * C * N, m0 + wm * (BM / 2), rows,
      n0 + wn * (SWIGLU ? BN / 4 : BN / 2), N, lane);
}

// ---------------------------------------------------------------------------
// bf16 matrix-core GEMM with the operands brought into LDS by the buffer
// unit itself (buffer_load_dwordx4 ... lds), bypassing registers. 256 x 256
// block of NW waves: with 4, one per SIMD, 2 x 2 waves of 128 x 128 (4 x 4
// v_mfma_f32_32x32x16_bf16 tiles); with 8, two per SIMD, 2 x 4 waves of
// 128 x 64 (4 x 2 tiles), so while one wave of a SIMD waits at a barrier or
// on its DMA the other's matrix work keeps the SIMD busy (the block tile, and
// with it the LDS and L2 traffic per flop, stays that of 256 x 256). K in
// 64-wide stages (every row a whole 128-byte line) through two LDS slots:
// stage k + 1 streams in while stage k feeds the matrix cores.
// Needs K % 128 == 0.
// LDS rows are 64 elements (eight 16-byte chunks); chunk c of row r sits at
// c ^ ((r / 2) % 8), so 16 lanes reading 16 consecutive rows hit 16 distinct
// bank groups. One DMA instruction of a wave fills 8 rows (1 KiB): lane L
// writes row L / 8, position L % 8, and so fetches the chunk that belongs
// there. Each slot is its own LDS array, so the compiler can tell the stages
// apart and the only waits on the DMA are the explicit ones below.
// ---------------------------------------------------------------------------
#define MOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define MOE_LDS_V4I16(p) ((__attribute__((address_space(3))) v4i16*)(p))

// s_waitcnt encodings (gfx9 family): vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum does not wait.
template <int VM>
__device__ inline void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
}

// With BT the B operand is stored K-major, [K][N] with N contiguous (B0 holds
// rows k < K0 and B1, if not NULL, rows K0 .. K - 1; K0 % 64 == 0). A stage of
// B is then 64 K rows x 256 columns in LDS, 16-byte chunk c of row k at
// position c ^ (4 (k % 4)), and each wave reads its fragments with
// ds_read_b64_tr_b16, which hands lane i of a 16-lane group element i % 4 of
// the piece that lane 4 q + i / 4 points at, as its element q: two such reads
// give a lane the eight consecutive K values of one column that the matrix
// core wants.
// With F32OUT the output is fp32 (out points at floats) and stored straight
// from the accumulators; kept and mtile_off may then be NULL: one group of C
// rows, all kept.
// With AT as well (weight gradients, out[e] = A_e^T B_e over each expert's
// kept rows), A is K-major too: element (k, m) of group e at
// A + e a_es + k lda + aoff + m, B's at B0 + e b_es + k N + n; group e
// contracts over kk[e] rows (rounded up to whole 64-row stages, the
// rows past kk[e] reading as zero), every group has C (= M) output rows, and
// kept and mtile_off are NULL.
template <bool SWIGLU, bool BT = false, bool F32OUT = false, bool AT = false, int NW = 4, int TM_ = 4,
          bool EARLY = true>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void gemm_bf16_dma_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
    bf16_t* __restrict__ out, const int32_t* __restrict__ kept, const int32_t* __restrict__ mtile_off,
    int E, int64_t C, int64_t K, int64_t N, int nt_count, const int32_t* __restrict__ wmap,
    float* __restrict__ part, int32_t* __restrict__ tick, int G, int64_t K0 = 0, int slices = 1,
    const int32_t* __restrict__ kk = nullptr, int64_t lda = 0, int64_t a_es = 0, int64_t aoff = 0,
    int64_t b_es = 0, bf16_t* __restrict__ gout = nullptr, bf16_t* __restrict__ uout = nullptr) {
  static_assert(!(SWIGLU && BT), "the K-major B operand serves the plain GEMM only");
  static_assert(!(F32OUT && (SWIGLU || BT)), "fp32 output serves the plain GEMM only");
  static_assert(!AT || (BT && !F32OUT), "a K-major A comes with a K-major B");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(TM_ == 4 || (TM_ == 5 && NW == 8 && !AT && !F32OUT), "320-row blocks: 8 waves, row-major A");
  // NW = 4: one wave per SIMD, 2 x 2 waves of 128 x 128. NW = 8: two waves per
  // SIMD, 2 x 4 waves of (32 TM) x 64, so one wave's matrix work covers the
  // other's barrier and DMA waits. TM = 5 makes the block 320 rows tall.
  constexpr int TM = TM_, BM = 64 * TM, BN = 256, BK = 64, TN = NW == 4 ? 4 : 2;
  constexpr int WNC = NW / 2;                   // waves along N
  constexpr int NTHR = NW * 64;
  constexpr int CH = BK / 8;                    // 16-byte chunks per LDS row
  constexpr int BNO = SWIGLU ? BN / 2 : BN;
  constexpr int PWA = BM / 8 / NW, PWB = BN / 8 / NW;  // 8-row DMA blocks per wave: A, B
  __shared__ uint4 As0[BM * CH], As1[BM * CH];
  __shared__ uint4 Bs0[BN * CH], Bs1[BN * CH];
  __shared__ int arrival;

  // With AT (no split round) the launch may hold fewer blocks than tiles: each
  // block then takes tile ids bid, bid + gridDim.x, ... (one XCD's, in order)
  // until its XCD's tiles run out.
  constexpr bool PERSIST = AT && kPersistAt;
  for (int64_t bid = blockIdx.x;; bid += gridDim.x) {
  Work wk;
  if (!work_of_block<BM>(mtile_off, E, nt_count, K / BK, G, &wk, C, slices, bid, AT ? nullptr : kept)) return;
  const int e = __builtin_amdgcn_readfirstlane(wk.e);
  const int m0 = __builtin_amdgcn_readfirstlane(wk.m0);
  const int nt = __builtin_amdgcn_readfirstlane(wk.nt);
  const int split = __builtin_amdgcn_readfirstlane(wk.s);
  const int chunk = __builtin_amdgcn_readfirstlane(wk.c);
  const int ti = __builtin_amdgcn_readfirstlane(wk.ti);
  const int kr_e = AT ? __builtin_amdgcn_readfirstlane(kk[e]) : 0;  // rows this group contracts over
  const int64_t kb = __builtin_amdgcn_readfirstlane(static_cast<int>(wk.kb));  // stages [kb, ke): even
  // with AT, whole 64-row stages over the group's kk[e] rows (an odd count ends
  // with a single stage)
  const int64_t ke = AT ? (kr_e + BK - 1) / BK : __builtin_amdgcn_readfirstlane(static_cast<int>(wk.ke));
  // rows of this tile end at r1 (its share of the expert's kept rows); those
  // past it belong to the next tile: never multiplied, loaded or stored here
  const int rows = __builtin_amdgcn_readfirstlane(
      min(kept ? bucket_rows(kept, e, C) : static_cast<int>(C), wk.r1));
  const int64_t n0 = static_cast<int64_t>(nt) * BNO;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // rows past kept (padding) read as zero without a memory access; with AT,
  // K rows past kk[e]
  const auto ra_src = AT ? buffer_rsrc(A + static_cast<int64_t>(e) * a_es, static_cast<uint32_t>(kr_e * lda * 2))
                         : buffer_rsrc(A + static_cast<int64_t>(e) * C * K,
                                       static_cast<uint32_t>(min(static_cast<int64_t>(rows), C) * K * 2));
  // B rows 0..127 of a SwiGLU block are gate rows, 128..255 up rows: the first
  // half of the waves load the first half
  const bf16_t* bbase = (SWIGLU && wave >= NW / 2) ? B1 : B0;
  const int we = wmap ? __builtin_amdgcn_readfirstlane(wmap[e]) : e;  // expert whose weights this row tile uses
  const int64_t kb0 = BT ? K0 : K;  // K rows held by B0
  const auto rb_src = AT ? buffer_rsrc(B0 + static_cast<int64_t>(e) * b_es, static_cast<uint32_t>(kr_e * N * 2))
                         : buffer_rsrc(bbase + static_cast<int64_t>(we) * N * kb0,
                                       static_cast<uint32_t>(N * kb0 * 2));
  const auto rb_src1 = buffer_rsrc(BT && B1 ? B1 + static_cast<int64_t>(we) * N * (K - K0) : B0,
                                   BT && B1 ? static_cast<uint32_t>(N * (K - K0) * 2) : 0u);
  // fixed sizes (a size that depends on the template parameters makes the host
  // pass drop the kernel); PWA, PWB <= 8
  uint32_t a_voff[8], b_voff[8];
#pragma unroll
  for (int i = 0; i < PWA; ++i) {
    const int row = (wave * PWA + i) * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((row >> 1) & 7);  // the chunk stored at position lane % 8
    if constexpr (AT) {  // as B below: K rows 2 u and 2 u + 1 of the stage, 32 positions each
      const int kr = (wave * PWA + i) * 2 + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (kr & 3));
      const int64_t am = m0 + c * 8;
      a_voff[i] = am < C ? static_cast<uint32_t>((kr * lda + aoff + am) * 2) : 0x80000000u;
    } else {
      a_voff[i] = static_cast<uint32_t>((m0 + row) * K * 2 + ch * 16);  // rows past kept read as zero
    }
  }
#pragma unroll
  for (int i = 0; i < PWB; ++i) {
    const int row = (wave * PWB + i) * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((row >> 1) & 7);
    if constexpr (BT) {
      // one instruction fills K rows 2 u and 2 u + 1 of the stage (u = wave * PWB + i), 32 positions each
      const int kr = (wave * PWB + i) * 2 + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (kr & 3));  // the chunk stored at position lane % 32
      const int64_t bn = n0 + c * 8;
      b_voff[i] = bn < N ? static_cast<uint32_t>((kr * N + bn) * 2) : 0x80000000u;
    } else {
      const int64_t bn = n0 + (SWIGLU ? (row % (BN / 2)) : row);
      b_voff[i] = bn < N ? static_cast<uint32_t>(bn * K * 2 + ch * 16) : 0x80000000u;
    }
  }
  auto dma = [&](uint4* as, uint4* bs, int64_t ks) {  // ks: stage number
    const uint32_t soff = static_cast<uint32_t>(ks * BK * 2);
    const uint32_t asoff = AT ? static_cast<uint32_t>(ks * BK * lda * 2) : soff;
#pragma unroll
    for (int i = 0; i < PWA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_src, MOE_LDS(as + (wave * PWA + i) * 8 * CH), 16,
                                               a_voff[i], asoff, 0, 0);
    if constexpr (BT) {
      const bool second = !AT && ks * BK >= K0;  // uniform: K0 is a multiple of the stage depth
      const auto rb = second ? rb_src1 : rb_src;
      const uint32_t bsoff = static_cast<uint32_t>((second ? ks * BK - K0 : ks * BK) * N * 2);
#pragma unroll
      for (int i = 0; i < PWB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, MOE_LDS(bs + (wave * PWB + i) * 8 * CH), 16, b_voff[i],
                                                 bsoff, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < PWB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb_src, MOE_LDS(bs + (wave * PWB + i) * 8 * CH), 16,
                                                 b_voff[i], soff, 0, 0);
    }
  };

  const int wm = wave / WNC, wn = wave % WNC;
  const int lr = lane & 31, lk = lane >> 5;
  int a_row[TM], b_row[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row[i] = (wm * (BM / 2) + i * 32 + lr) * CH;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int br = SWIGLU ? ((j < TN / 2) ? (wn * (TN / 2 * 32) + j * 32)
                                          : (BN / 2 + wn * (TN / 2 * 32) + (j - TN / 2) * 32))
                          : (wn * (TN * 32) + j * 32);
    b_row[j] = (br + lr) * CH;
  }
  // K-major B: byte offset, within a stage, of this lane's first 8-byte piece
  // of fragment j (sub-step 0, K values 0..3 of its column group)
  int bt_off[TN], at_off[TM];
  if constexpr (BT) {
    const int g = lane >> 4, jj = lane & 15;
    const int kr = 8 * (g >> 1) + (jj >> 2);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int nl = wn * (TN * 32) + j * 32 + 16 * (g & 1) + 4 * (jj & 3);
      bt_off[j] = kr * (BN * 2) + (((nl >> 3) ^ (4 * (jj >> 2))) * 16) + (nl & 7) * 2;
    }
    if constexpr (AT) {  // the same for the 32-row blocks of A (BM == BN)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int ml = wm * (BM / 2) + i * 32 + 16 * (g & 1) + 4 * (jj & 3);
        at_off[i] = kr * (BM * 2) + (((ml >> 3) ^ (4 * (jj >> 2))) * 16) + (ml & 7) * 2;
      }
    }
  }
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // A wave whose rows lie partly past the tile's kept rows multiplies only
  // its first TA of TM 32-row blocks (rows past kept are never stored); it
  // still issues its share of every stage's loads and takes every barrier.
  // Raised wave priority over each stage's matrix run, 320-row blocks only:
  // there the two waves of a SIMD multiply unequal row counts (5 and 3 blocks
  // at DeepSeek-V3's fill), and favouring the wave that is multiplying took
  // that GEMM 1 from 4.29 to 3.97 ms; on 256-row blocks it measured neutral
  // to slightly slower.
  constexpr bool PRIO = NW == 8 && TM == 5;
  const int live_rows = rows - m0 - wm * (BM / 2);
  const int ta = __builtin_amdgcn_readfirstlane(live_rows <= 0 ? 0 : min(TM, (live_rows + 31) / 32));
  const int rsw = (lr >> 1) & 7;
  auto kloop = [&](auto ta_c) {
    constexpr int TA = decltype(ta_c)::value;
    constexpr int NMFMA = TA * TN, NFRAG = TA > 0 ? (AT ? 2 : 1) * TA + (BT ? 2 : 1) * TN : 1;
    bf16x8 fa[2][TM], fb[2][TN];
    auto tr_pair = [](const char* p) {  // 8 consecutive K values of one column of a K-major stage
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MOE_LDS_V4I16(p));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MOE_LDS_V4I16(p + 4 * BN * 2));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto fload = [&](const uint4* as, const uint4* bs, int ks, int slot) {
      if constexpr (TA > 0) {
        const int pc = (ks * 2 + lk) ^ rsw;
        if constexpr (AT) {
          const char* abase = reinterpret_cast<const char*>(as) + ks * 16 * (BM * 2);
#pragma unroll
          for (int i = 0; i < TA; ++i) fa[slot][i] = tr_pair(abase + at_off[i]);
        } else {
#pragma unroll
          for (int i = 0; i < TA; ++i) fa[slot][i] = *reinterpret_cast<const bf16x8*>(&as[a_row[i] + pc]);
        }
        if constexpr (BT) {
          const char* base = reinterpret_cast<const char*>(bs) + ks * 16 * (BN * 2);
#pragma unroll
          for (int j = 0; j < TN; ++j) fb[slot][j] = tr_pair(base + bt_off[j]);
        } else {
#pragma unroll
          for (int j = 0; j < TN; ++j) fb[slot][j] = *reinterpret_cast<const bf16x8*>(&bs[b_row[j] + pc]);
        }
      }
    };
    auto mfmas = [&](int slot) {
#pragma unroll
      for (int i = 0; i < TA; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
    };
    // interleave the next fragments' LDS reads with this step's matrix work
    auto interleave = [&](auto reads_first) {
      if constexpr (TA == TM)
        interleave_groups<NMFMA, NFRAG, decltype(reads_first)::value>(std::make_integer_sequence<int, NFRAG>{});
    };
    // Stage k is in (as, bs). With EARLY, stage k + 1 is already on its way
    // into (an, bn_); once every wave has read its last fragments of stage k
    // and stage k + 1 has landed (one barrier), stage k + 2 is requested into
    // (as, bs) at once, a sub-step before the matrix work of stage k ends, so
    // each stage's loads have a stage and a quarter of matrix work to arrive.
    // Without EARLY, stage k + 1 is requested as stage k starts (one stage).
    auto stage = [&](auto has_next, auto has_next2, uint4* as, uint4* bs, uint4* an, uint4* bn_, int64_t k) {
      if constexpr (!EARLY && decltype(has_next)::value) dma(an, bn_, k + 1);
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);  // the matrix run goes first
      fload(as, bs, 1, 1);
      mfmas(0);
      interleave(std::false_type{});
      fload(as, bs, 2, 0);
      mfmas(1);
      interleave(std::false_type{});
      fload(as, bs, 3, 1);
      mfmas(0);
      interleave(std::false_type{});
      if constexpr (PRIO) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
      }
      if constexpr (decltype(has_next)::value) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm0<0>();            // own DMA of stage k + 1 landed, reads of stage k done ...
        __builtin_amdgcn_s_barrier();  // ... and everyone else's
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (EARLY && decltype(has_next2)::value) dma(as, bs, k + 2);
        fload(an, bn_, 0, 0);
      }
      mfmas(1);
      interleave(std::true_type{});
    };
    using T_ = std::true_type;
    using F_ = std::false_type;

    dma(As0, Bs0, kb);
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    // ke - kb is even and positive, or, with AT, positive: a stage past the
    // group's rows (one of an odd count's) is requested at most once and reads
    // zeros (its rows lie past kk[e], outside the buffer ranges)
    if constexpr (EARLY) dma(As1, Bs1, kb + 1);
    fload(As0, Bs0, 0, 0);
    int64_t k = kb;
    for (; k + 2 < ke; k += 2) {  // then k + 3 < ke as well, or (AT, odd count) k + 3 == ke
      stage(T_{}, T_{}, As0, Bs0, As1, Bs1, k);
      stage(T_{}, T_{}, As1, Bs1, As0, Bs0, k + 1);
    }
    stage(T_{}, F_{}, As0, Bs0, As1, Bs1, k);
    // an odd count (AT) has no stage k + 1: its zeros are waited for above
    // but not multiplied
    if (!AT || k + 1 < ke) stage(F_{}, F_{}, As1, Bs1, As0, Bs0, k + 1);
  };
  if (ke > kb) {  // with AT a group that kept no row contracts over nothing: its block is zero
    if (ta >= TM || (TM == 4 && ta == 3))
      kloop(std::integral_constant<int, TM>{});
    else if (TM == 5 && ta == 4)
      kloop(std::integral_constant<int, TM == 5 ? 4 : TM>{});
    else if (TM == 5 && ta == 3)
      kloop(std::integral_constant<int, TM == 5 ? 3 : TM>{});
    else if (ta == 2)
      kloop(std::integral_constant<int, 2>{});
    else if (ta == 1)
      kloop(std::integral_constant<int, 1>{});
    else
      kloop(std::integral_constant<int, 0>{});
  }

  if (split > 1) {
    // Chunk of a split tile: publish the fp32 partial (thread t writes its
    // 64 float4s at [g][t], coalesced), count the arrival; the last of the s
    // blocks to arrive adds the s partials in chunk order, so the sum does
    // not depend on which block came last.
    constexpr int NG = TM * TN * 4;  // float4 groups per thread
    float4* mine = reinterpret_cast<float4*>(part) + static_cast<int64_t>(ti * split + chunk) * NG * NTHR;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          mine[((i * TN + j) * 4 + q) * NTHR + tid] =
              float4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    __threadfence();
    __syncthreads();
    if (tid == 0) arrival = atomicAdd(&tick[ti], 1);
    __syncthreads();
    if (arrival != split - 1) return;
    if (tid == 0) tick[ti] = 0;  // every arrival is in: the counter is ready for the next launch
    __threadfence();
    // every partial, this block's own included, is read back in chunk order;
    // a group's s loads are in flight together (a load-add chain would wait
    // out the memory latency once per load)
    const float4* first =
        reinterpret_cast<const float4*>(part) + static_cast<int64_t>(ti * split) * NG * NTHR + tid;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int g = (i * TN + j) * 4 + q;
          float4 v[kMaxSplit];
#pragma unroll
          for (int c = 0; c < kMaxSplit; ++c)
            if (c < split) v[c] = first[(static_cast<int64_t>(c) * NG + g) * NTHR];
          float4 t = v[0];
#pragma unroll
          for (int c = 1; c < kMaxSplit; ++c)
            if (c < split) {
              t.x += v[c].x;
              t.y += v[c].y;
              t.z += v[c].z;
              t.w += v[c].w;
            }
          acc[i][j][4 * q] = t.x;
          acc[i][j][4 * q + 1] = t.y;
          acc[i][j][4 * q + 2] = t.z;
          acc[i][j][4 * q + 3] = t.w;
        }
  }

  if constexpr (F32OUT) {  // lanes 0-31 and 32-63 each store 32 consecutive floats of one row
    // with K slices, slice c of [slices][C][N]
    float* o = reinterpret_cast<float*>(out) + static_cast<int64_t>(e) * C * N +
               (slices > 1 ? static_cast<int64_t>(chunk) * C * N : 0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = m0 + wm * (BM / 2) + i * 32 + 8 * (q >> 2) + 4 * lk + (q & 3);
          const int64_t c = n0 + wn * (TN * 32) + j * 32 + lr;
          if (r < rows && c < N) o[r * N + c] = acc[i][j][q];
        }
    return;
  }
  // the stage buffers are free: one per wave for the epilogue (half of one with 8 waves)
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  const int sb = wave / (NW / 4);
  constexpr int EB = BN * CH * 16 / (NW / 4);  // bytes per wave (A slots are at least as large)
  char* eb = reinterpret_cast<char*>(sb == 0 ? As0 : sb == 1 ? As1 : sb == 2 ? Bs0 : Bs1) + (wave % (NW / 4)) * EB;
  // K-major (BT) instantiations run only in the backward pass, where non-temporal stores
  // measured 0.2-2% faster end to end; the forward GEMMs measured faster with plain stores
  store_wave_tile<TM, TN, SWIGLU, EB, true, BT>(
      acc, eb, out + static_cast<int64_t>(e) * C * N, m0 + wm * (BM / 2), rows,
      n0 + wn * (SWIGLU ? TN * 16 : TN * 32), N, lane);
  if constexpr (SWIGLU) {
    // g and u themselves, rounded, when kept for the backward: the gate
    // accumulators (column blocks 0 .. TN/2) and the up ones, at h's columns
    if (gout) {
      f32x16 half[TM][TN / 2];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) half[i][j] = acc[i][j];
      store_wave_tile<TM, TN / 2, false, EB, true, false>(half, eb, gout + static_cast<int64_t>(e) * C * N,
                                                          m0 + wm * (BM / 2), rows, n0 + wn * TN * 16, N, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) half[i][j] = acc[i][j + TN / 2];
      store_wave_tile<TM, TN / 2, false, EB, true, false>(half, eb, uout + static_cast<int64_t>(e) * C * N,
                                                          m0 + wm * (BM / 2), rows, n0 + wn * TN * 16, N, lane);
    }
  }
  if constexpr (!PERSIST) return;
  __syncthreads();  // every wave's staging reads are done before the next tile's DMA
  }
}

// ---------------------------------------------------------------------------
// 128 x 256 variant for two work-groups per CU: K in 32-wide stages (64-byte
// LDS rows) through two slots, 48 KiB in all, so a second work-group's matrix
// work covers this one's barriers, DMA waits and epilogue. 4 waves (2 x 2) of
// 64 x 128, each as 2 x 4 v_mfma_f32_32x32x16_bf16 tiles. One DMA instruction
// of a wave fills 16 rows (lane L: row L / 4, position L % 4); chunk c of row
// r sits at position c ^ ((r / 4) % 4), so the 16 lanes of a fragment read
// (16 consecutive rows) hit distinct banks. Needs K % 64 == 0.
// ---------------------------------------------------------------------------
template <bool SWIGLU>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_bf16_dma_m128_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
    bf16_t* __restrict__ out, const int32_t* __restrict__ kept, const int32_t* __restrict__ mtile_off,
    int E, int64_t C, int64_t K, int64_t N, int nt_count, const int32_t* __restrict__ wmap) {
  constexpr int BM = 128, BN = 256, BK = 32, TM = 2, TN = 4;
  constexpr int CH = BK / 8;                    // 16-byte chunks per LDS row
  constexpr int BNO = SWIGLU ? BN / 2 : BN;
  constexpr int A_PW = BM / 16 / 4;             // 16-row DMA blocks per wave: A (2), B (4)
  constexpr int B_PW = BN / 16 / 4;
  constexpr int NMFMA = TM * TN, NFRAG = TM + TN;
  __shared__ uint4 As0[BM * CH], As1[BM * CH];
  __shared__ uint4 Bs0[BN * CH], Bs1[BN * CH];

  int e, m0, nt;
  if (!tile_of_block<BM>(mtile_off, E, nt_count, &e, &m0, &nt)) return;
  e = __builtin_amdgcn_readfirstlane(e);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  nt = __builtin_amdgcn_readfirstlane(nt);
  const int rows = __builtin_amdgcn_readfirstlane(bucket_rows(kept, e, C));
  const int64_t n0 = static_cast<int64_t>(nt) * BNO;
  const int64_t nk = K / BK;  // even, at least 2

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // rows past kept (padding) read as zero without a memory access
  const auto ra_src = buffer_rsrc(A + static_cast<int64_t>(e) * C * K,
                                  static_cast<uint32_t>(min(static_cast<int64_t>(rows), C) * K * 2));
  // B rows 0..127 of a SwiGLU block are gate rows, 128..255 up rows: waves 0-1
  // load the first half, waves 2-3 the second
  const bf16_t* bbase = (SWIGLU && wave >= 2) ? B1 : B0;
  const int we = wmap ? __builtin_amdgcn_readfirstlane(wmap[e]) : e;  // expert whose weights this row tile uses
  const auto rb_src = buffer_rsrc(bbase + static_cast<int64_t>(we) * N * K, static_cast<uint32_t>(N * K * 2));
  uint32_t a_voff[A_PW], b_voff[B_PW];
#pragma unroll
  for (int i = 0; i < A_PW; ++i) {
    const int row = (wave * A_PW + i) * 16 + (lane >> 2);
    const int ch = (lane & 3) ^ ((row >> 2) & 3);  // the chunk stored at position lane % 4
    a_voff[i] = static_cast<uint32_t>((m0 + row) * K * 2 + ch * 16);  // rows past kept read as zero
  }
#pragma unroll
  for (int i = 0; i < B_PW; ++i) {
    const int row = (wave * B_PW + i) * 16 + (lane >> 2);
    const int ch = (lane & 3) ^ ((row >> 2) & 3);
    const int64_t bn = n0 + (SWIGLU ? (row % (BN / 2)) : row);
    b_voff[i] = bn < N ? static_cast<uint32_t>(bn * K * 2 + ch * 16) : 0x80000000u;
  }
  auto dma = [&](uint4* as, uint4* bs, int64_t ks) {  // ks: stage number
    const uint32_t soff = static_cast<uint32_t>(ks * BK * 2);
#pragma unroll
    for (int i = 0; i < A_PW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_src, MOE_LDS(as + (wave * A_PW + i) * 16 * CH), 16, a_voff[i],
                                               soff, 0, 0);
#pragma unroll
    for (int i = 0; i < B_PW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb_src, MOE_LDS(bs + (wave * B_PW + i) * 16 * CH), 16, b_voff[i],
                                               soff, 0, 0);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
  int a_row[TM], b_row[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row[i] = (wm * (BM / 2) + i * 32 + lr) * CH;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int br = SWIGLU ? ((j < TN / 2) ? (wn * (BN / 4) + j * 32) : (BN / 2 + wn * (BN / 4) + (j - TN / 2) * 32))
                          : (wn * (BN / 2) + j * 32);
    b_row[j] = (br + lr) * CH;
  }
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  bf16x8 fa[2][TM], fb[2][TN];
  const int rsw = (lr >> 2) & 3;
  auto fload = [&](const uint4* as, const uint4* bs, int ks, int slot) {
    const int pc = (ks * 2 + lk) ^ rsw;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[slot][i] = *reinterpret_cast<const bf16x8*>(&as[a_row[i] + pc]);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[slot][j] = *reinterpret_cast<const bf16x8*>(&bs[b_row[j] + pc]);
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
  };
  auto interleave = [&]() {  // 8 matrix ops with the 6 fragment reads between them
#pragma unroll
    for (int g = 0; g < NFRAG; ++g) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMFMA - NFRAG, 0);
  };
  // Stage k in (as, bs); stage k + 1 goes to (an, bn_) unless this is the last.
  auto stage = [&](auto has_next, const uint4* as, const uint4* bs, uint4* an, uint4* bn_, int64_t k) {
    if constexpr (decltype(has_next)::value) dma(an, bn_, k + 1);
    fload(as, bs, 1, 1);
    mfmas(0);
    interleave();
    if constexpr (decltype(has_next)::value) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_lgkm0<0>();            // own DMA of stage k + 1 landed, reads of stage k done ...
      __builtin_amdgcn_s_barrier();  // ... and everyone else's
      __builtin_amdgcn_sched_barrier(0);
      fload(an, bn_, 0, 0);
    }
    mfmas(1);
    interleave();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  dma(As0, Bs0, 0);
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  fload(As0, Bs0, 0, 0);
  int64_t k = 0;
  for (; k + 2 < nk; k += 2) {
    stage(T_{}, As0, Bs0, As1, Bs1, k);
    stage(T_{}, As1, Bs1, As0, Bs0, k + 1);
  }
  stage(T_{}, As0, Bs0, As1, Bs1, k);
  stage(F_{}, As1, Bs1, As0, Bs0, k + 1);

  // the stage buffers are free: an 8 KiB half of a B slot per wave for the epilogue
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  char* eb = reinterpret_cast<char*>(wave < 2 ? Bs0 : Bs1) + (wave & 1) * (BN * CH * 8);
  store_wave_tile<TM, TN, SWIGLU, BN * CH * 8, false>(acc, eb, out + static_cast<int64_t>(e) * C * N,
                                                       m0 + wm * (BM / 2), rows,
                                                       n0 + wn * (SWIGLU ? BN / 4 : BN / 2), N, lane);
}

// ---------------------------------------------------------------------------
// Few rows per expert (decode): the run is a stream of each touched expert's
// weights, each element used by at most 16 rows. A work-group takes one
// expert's rows (16 at most) and 64 output columns; each wave owns 16 columns
// as 16 x 16 v_mfma_f32_16x16x32_bf16 tiles (for SWIGLU a gate and an up
// tile), K in steps of 32. Weights go straight from HBM to registers, eight
// K steps in flight per lane; the few activation rows come from L2.
// Operand lane layout: lane l holds row (l % 16), K elements 8*(l/16) .. +8;
// accumulator element r of lane l is row 4*(l/16) + r, column l % 16.
// ---------------------------------------------------------------------------
constexpr int kSkinnyRows = 16;

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_bf16_skinny_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
    bf16_t* __restrict__ out, const int32_t* __restrict__ kept, const int32_t* __restrict__ mtile_off,
    int E, int64_t C, int64_t K, int64_t N, int nch, const int32_t* __restrict__ wmap) {
  constexpr int U = 8;  // K steps in flight
  const int mt = blockIdx.x / nch;
  const int nc = blockIdx.x - mt * nch;
  if (mt >= mtile_off[E]) return;
  const int e = __builtin_amdgcn_readfirstlane(owner_expert(mtile_off, E, mt));
  const int m0 = __builtin_amdgcn_readfirstlane((mt - mtile_off[e]) * kSkinnyRows);
  const int rows = __builtin_amdgcn_readfirstlane(bucket_rows(kept, e, C));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col0 = static_cast<int64_t>(nc) * 64 + wave * 16;
  if (col0 >= N) return;
  const int kg = (lane >> 4) * 8;
  const int arow = m0 + (lane & 15);
  const bool a_in = arow < rows;
  const bf16_t* ap = A + (static_cast<int64_t>(e) * C + (a_in ? arow : 0)) * K + kg;
  const int64_t bcol = min(col0 + (lane & 15), N - 1);
  const int64_t we = wmap ? __builtin_amdgcn_readfirstlane(wmap[e]) : e;
  const bf16_t* b0p = B0 + (we * N + bcol) * K + kg;
  const bf16_t* b1p = SWIGLU ? B1 + (we * N + bcol) * K + kg : nullptr;

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int64_t nk = K / 32;  // K is a multiple of 32 here
  int64_t ks = 0;
  for (; ks + U <= nk; ks += U) {
    bf16x8 a[U], b0[U], b1[U];
    // one matrix at a time: consecutive loads of a lane fall in the same
    // 128-byte lines (4 lanes x 16 bytes per step of 32), so each weight line
    // is requested by back-to-back loads
#pragma unroll
    for (int u = 0; u < U; ++u) b0[u] = *reinterpret_cast<const bf16x8*>(b0p + (ks + u) * 32);
    if (SWIGLU) {
#pragma unroll
      for (int u = 0; u < U; ++u) b1[u] = *reinterpret_cast<const bf16x8*>(b1p + (ks + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = a_in ? *reinterpret_cast<const bf16x8*>(ap + (ks + u) * 32) : bf16x8{};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b0[u], acc0, 0, 0, 0);
      if (SWIGLU) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b1[u], acc1, 0, 0, 0);
    }
  }
  for (; ks < nk; ++ks) {
    const bf16x8 b0v = *reinterpret_cast<const bf16x8*>(b0p + ks * 32);
    const bf16x8 av = a_in ? *reinterpret_cast<const bf16x8*>(ap + ks * 32) : bf16x8{};
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b0v, acc0, 0, 0, 0);
    if (SWIGLU) {
      const bf16x8 b1v = *reinterpret_cast<const bf16x8*>(b1p + ks * 32);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b1v, acc1, 0, 0, 0);
    }
  }
  const int64_t col = col0 + (lane & 15);
  if (col >= N) return;
  bf16_t* oute = out + static_cast<int64_t>(e) * C * N;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = m0 + 4 * (lane >> 4) + r;
    if (row < rows)
      oute[row * N + col] = f32_to_bf16(SWIGLU ? silu_bf16(acc0[r]) * acc1[r] : acc0[r]);
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
                                                       int E, int64_t C, int64_t K, int64_t N,
                                                       const int32_t* __restrict__ wmap) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr int NB = SWIGLU ? 2 : 1;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[NB][BK][BN + 4];

  const int mt = blockIdx.x;
  if (mt >= mtile_off[E]) return;
  const int e = owner_expert(mtile_off, E, mt);
  const int m0 = (mt - mtile_off[e]) * BM;
  const int rows = bucket_rows(kept, e, C);
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const float* Ae = A + static_cast<int64_t>(e) * C * K;
  const int64_t we = wmap ? wmap[e] : e;
  const float* Bp[2] = {B0 + we * N * K, SWIGLU ? B1 + we * N * K : nullptr};

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

// Block shape of the bf16 kernel: 256 x 256 once experts hold enough rows to
// fill it, else 128 x 128.
constexpr int kBigTileMinC = 512;
constexpr int kBigTileMinCGateUp = 256;

// Row tiles of the skinny kernel when every expert holds this few rows.
constexpr int kSkinnyMaxC = kSkinnyRows;

size_t split_k_bytes() {
  return static_cast<size_t>(kSplitUnits) * kSplitTileElems * sizeof(float) + kSplitUnits * sizeof(int32_t);
}

SplitK split_k_carve(void* base) {
  if (!base) return SplitK{nullptr, nullptr};
  auto* p = static_cast<float*>(base);
  return SplitK{p, reinterpret_cast<int32_t*>(p + static_cast<size_t>(kSplitUnits) * kSplitTileElems)};
}

int grouped_gemm_bm(bool bf16, int64_t C) {
  if (!bf16) return 64;
  if (C <= kSkinnyMaxC) return kSkinnyRows;
  return C >= kBigTileMinC ? 256 : 128;
}

// The backward GEMMs that contract over d (g and u recomputed, dh, dX). Each
// weight tile streams once per row tile: from 256 rows of capacity on, one
// 256-row tile per expert (its padding rows cost no matrix work and no loads)
// beats two 128-row tiles that each stream the weights. With 256 < C <= 320 a
// 256-row tile would leave most experts a second, nearly empty tile that
// streams the same weights again; one 320-row tile covers every expert (needs
// K % 128 == 0, as the 256-row tile does). Larger C take 320-row tiles when
// K >= 4096 (Mixtral's backward 8.17 -> 7.95 ms); at the skewed workload's
// K = 2048 they cost 12%.
int grouped_gemm_bm_contract_d(bool bf16, int64_t C, int64_t K) {
  if (!bf16) return 64;
  if (C <= kSkinnyMaxC) return kSkinnyRows;
  if (C > 256 && K % 128 == 0 && (C <= 320 || K >= 4096)) return 320;
  return C >= kBigTileMinCGateUp ? 256 : 128;
}

// GEMM 1 in the forward pass: the same rule. At Mixtral's C = 1280 four
// 320-row tiles fit exactly, and the nearly empty fifth 256-row tile of an
// expert just over 1024 rows is gone (gate/up 1.77 -> 1.72 ms). At K = 2048
// the skewed workload gained 3% from them but its replicated layout lost 15%.
int grouped_gemm_bm_gate_up(bool bf16, int64_t C, int64_t K) { return grouped_gemm_bm_contract_d(bf16, C, K); }

// GEMM 2 in the forward pass: 320-row tiles for 256 < C <= 320 as above, and
// for larger C when K >= 4096 (Mixtral's down GEMM 1.05 -> 0.89 ms: 512
// tiles, two whole rounds, instead of 576). With short K they lost (the
// skewed workload's K = 1408: 0.227 -> 0.361 ms).
int grouped_gemm_bm_down(bool bf16, int64_t C, int64_t K) {
  if (bf16 && C > 256 && K % 128 == 0 && (C <= 320 || K >= 4096)) return 320;
  return grouped_gemm_bm(bf16, C);
}

namespace {

template <bool SWIGLU>
hipError_t launch_skinny(const void* a, const void* b0, const void* b1, void* out, const int32_t* kept,
                         const int32_t* mtile_off, int E, int64_t C, int64_t K, int64_t N, const int32_t* wmap,
                         hipStream_t s) {
  const int64_t nch = ceil_div(N, 64);
  const int64_t blocks = E * ceil_div(C, kSkinnyRows) * nch;
  gemm_bf16_skinny_kernel<SWIGLU><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
      static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(b0), static_cast<const bf16_t*>(b1),
      static_cast<bf16_t*>(out), kept, mtile_off, E, C, K, N, static_cast<int>(nch), wmap);
  return hipGetLastError();
}

// Work-groups of the 256 x 256 kernel resident at once (one per CU), rounded
// down to whole rounds over the 8 XCDs; 0 if unknown (no split).
int resident_groups() {
  static std::atomic<int> cached[64];  // per device; 0 = not yet asked
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int g = cached[dev].load(std::memory_order_relaxed);
  if (g == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g = std::max(8, std::min(cus, kSplitUnits) / 8 * 8);
    cached[dev].store(g, std::memory_order_relaxed);
  }
  return g;
}

// Waves per work-group of the 256 x 256 kernel: row-major GEMMs, fp32-output
// row GEMM (router scores), K-major B (backward dh, dX), K-major A and B
// (weight gradients).
constexpr int kDmaWaves = 8;
constexpr int kRowsF32Waves = 8;
constexpr int kKmajorWaves = 8;
constexpr int kTnWaves = 8;

template <int BM, int BN, bool SWIGLU>
hipError_t launch_bf16(const void* a, const void* b0, const void* b1, void* out, const int32_t* kept,
                       const int32_t* mtile_off, int E, int64_t C, int64_t K, int64_t N, const int32_t* wmap,
                       hipStream_t s, const SplitK* sk = nullptr, void* gout = nullptr, void* uout = nullptr) {
  // only the LDS-DMA kernel also writes the SwiGLU GEMM's g and u
  if ((gout || uout) && !(SWIGLU && (BM == 320 || BM == 256) && BN == 256 && K % 128 == 0))
    return hipErrorInvalidValue;
  auto* pg = static_cast<bf16_t*>(gout);
  auto* pu = static_cast<bf16_t*>(uout);
  const int64_t mt_max = E * ceil_div(C, BM);  // upper bound of live row tiles
  const int64_t nt = ceil_div(N, SWIGLU ? BN / 2 : BN);
  int64_t blocks = ceil_div(mt_max * nt, 8) * 8;  // whole rounds over the 8 XCDs
  const auto* pa = static_cast<const bf16_t*>(a);
  const auto* pb0 = static_cast<const bf16_t*>(b0);
  const auto* pb1 = static_cast<const bf16_t*>(b1);
  auto* po = static_cast<bf16_t*>(out);
  if constexpr (BM == 320 && BN == 256) {
    if (K % 128) return hipErrorInvalidValue;  // callers pick this tile only for K % 128 == 0
    const int G = sk ? resident_groups() : 0;
    if (G > 0 && !sk->zeroed) {
      const hipError_t err = launch_fill_i32(sk->tick, G, 0, s);
      if (err != hipSuccess) return err;
    }
    if (G > 0) blocks += G;
    // Each stage's loads are requested a sub-step early, except for SwiGLU
    // over experts of 64 or more column tiles: there (d_ff = 14336, K = 4096)
    // the early request measured 2% slower, against 1-4% faster elsewhere.
    if (SWIGLU && nt >= 64)
      gemm_bf16_dma_kernel<SWIGLU, false, false, false, 8, 5, false>
          <<<dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s>>>(
          pa, pb0, pb1, po, kept, mtile_off, E, C, K, N, static_cast<int>(nt), wmap, G > 0 ? sk->part : nullptr,
          G > 0 ? sk->tick : nullptr, G, 0, 1, nullptr, 0, 0, 0, 0, pg, pu);
    else
      gemm_bf16_dma_kernel<SWIGLU, false, false, false, 8, 5><<<dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s>>>(
          pa, pb0, pb1, po, kept, mtile_off, E, C, K, N, static_cast<int>(nt), wmap, G > 0 ? sk->part : nullptr,
          G > 0 ? sk->tick : nullptr, G, 0, 1, nullptr, 0, 0, 0, 0, pg, pu);
  } else if constexpr (BM == 128 && BN == 256) {
    if (K % 64) return hipErrorInvalidValue;  // callers pick this tile only for K % 64 == 0
    gemm_bf16_dma_m128_kernel<SWIGLU><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
        pa, pb0, pb1, po, kept, mtile_off, E, C, K, N, static_cast<int>(nt), wmap);
  } else if constexpr (BM == 256 && BN == 256) {
    if (K % 128) {
      gemm_bf16_kernel<BM, BN, SWIGLU><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
          pa, pb0, pb1, po, kept, mtile_off, E, C, K, N, static_cast<int>(nt), wmap);
      return hipGetLastError();
    }
    const int G = sk ? resident_groups() : 0;
    if (G > 0 && !sk->zeroed) {
      const hipError_t err = launch_fill_i32(sk->tick, G, 0, s);
      if (err != hipSuccess) return err;
    }
    if (G > 0) blocks += G;  // the split round: at most G blocks beyond the whole tiles
    gemm_bf16_dma_kernel<SWIGLU, false, false, false, kDmaWaves>
        <<<dim3(static_cast<unsigned>(blocks)), dim3(kDmaWaves * 64), 0, s>>>(
        pa, pb0, pb1, po, kept, mtile_off, E, C, K, N, static_cast<int>(nt), wmap, G > 0 ? sk->part : nullptr,
        G > 0 ? sk->tick : nullptr, G, 0, 1, nullptr, 0, 0, 0, 0, pg, pu);
  } else {
    gemm_bf16_kernel<BM, BN, SWIGLU><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
        pa, pb0, pb1, po, kept, mtile_off, E, C, K, N, static_cast<int>(nt), wmap);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_rows_f32(const void* a, const void* b, int64_t M, int64_t K, int64_t N, int slices,
                                float* out, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (K % 128 || N % 8 || slices < 1 || slices > K / 128) return hipErrorInvalidValue;
  const int64_t nt = ceil_div(N, 256);
  const int64_t blocks = ceil_div(M, 256) * nt * slices;
  gemm_bf16_dma_kernel<false, false, true, false, kRowsF32Waves>
      <<<dim3(static_cast<unsigned>(blocks)), dim3(kRowsF32Waves * 64), 0, s>>>(
      static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(b), nullptr, reinterpret_cast<bf16_t*>(out),
      nullptr, nullptr, 1, M, K, N, static_cast<int>(nt), nullptr, nullptr, nullptr, 0, 0, slices);
  return hipGetLastError();
}

hipError_t launch_gemm_tn(const void* a, int64_t lda, int64_t a_es, int64_t aoff, const void* b, int64_t b_es,
                          const int32_t* kk, int E, int64_t M, int64_t N, void* out, hipStream_t s) {
  if (E == 0 || M == 0 || N == 0) return hipSuccess;
  if (M % 8 || N % 8 || lda % 8 || aoff % 8 || aoff + M > lda) return hipErrorInvalidValue;
  const int64_t nt = ceil_div(N, 256);
  int64_t blocks = ceil_div(E * ceil_div(M, 256) * nt, 8) * 8;
  if (kPersistAt) {  // one resident block per CU walks its XCD's tiles
    const int g = resident_groups();
    if (g > 0) blocks = std::min<int64_t>(blocks, g);
  }
  gemm_bf16_dma_kernel<false, true, false, true, kTnWaves>
      <<<dim3(static_cast<unsigned>(blocks)), dim3(kTnWaves * 64), 0, s>>>(
      static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(b), nullptr, static_cast<bf16_t*>(out), nullptr,
      nullptr, E, M, 0, N, static_cast<int>(nt), nullptr, nullptr, nullptr, 0, 0, 1, kk, lda, a_es, aoff, b_es);
  return hipGetLastError();
}

hipError_t launch_gemm_kmajor_b(const void* a, const int32_t* kept, const int32_t* mtile_off, const void* b0,
                                const void* b1, int64_t K0, int E, int64_t C, int64_t K, int64_t N, void* out,
                                hipStream_t s, const SplitK* sk, int bm) {
  if (E * C == 0) return hipSuccess;
  if (K % 128 || K0 % 64 || K0 <= 0 || K0 > K || (K0 < K && !b1) || N % 8 || (bm != 256 && bm != 320))
    return hipErrorInvalidValue;
  const int64_t mt_max = E * ceil_div(C, bm);
  const int64_t nt = ceil_div(N, 256);
  int64_t blocks = ceil_div(mt_max * nt, 8) * 8;
  const int G = sk ? resident_groups() : 0;
  if (G > 0 && !sk->zeroed) {
    const hipError_t err = launch_fill_i32(sk->tick, G, 0, s);
    if (err != hipSuccess) return err;
  }
  if (G > 0) blocks += G;
  const auto* pa = static_cast<const bf16_t*>(a);
  const auto* pb0 = static_cast<const bf16_t*>(b0);
  const auto* pb1 = static_cast<const bf16_t*>(b1);
  auto* po = static_cast<bf16_t*>(out);
  float* part = G > 0 ? sk->part : nullptr;
  int32_t* tick = G > 0 ? sk->tick : nullptr;
  if (bm == 320)
    gemm_bf16_dma_kernel<false, true, false, false, 8, 5><<<dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s>>>(
        pa, pb0, pb1, po, kept, mtile_off, E, C, K, N, static_cast<int>(nt), nullptr, part, tick, G, K0);
  else
    gemm_bf16_dma_kernel<false, true, false, false, kKmajorWaves>
        <<<dim3(static_cast<unsigned>(blocks)), dim3(kKmajorWaves * 64), 0, s>>>(
        pa, pb0, pb1, po, kept, mtile_off, E, C, K, N, static_cast<int>(nt), nullptr, part, tick, G, K0);
  return hipGetLastError();
}

bool gate_up_keeps_gu(bool bf16, int64_t C, int64_t d) {
  const int bm = grouped_gemm_bm_gate_up(bf16, C, d);
  return bf16 && (bm == 320 || bm == 256) && d % 128 == 0;
}

hipError_t launch_gemm_gate_up(const void* buckets, const int32_t* kept, const int32_t* mtile_off,
                               const void* wg, const void* wu, int E, int64_t C, int64_t d,
                               int64_t d_ff, bool bf16, void* h, hipStream_t s, const int32_t* wmap,
                               const SplitK* sk, void* g, void* u) {
  if ((g || u) && !(g && u && gate_up_keeps_gu(bf16, C, d))) return hipErrorInvalidValue;
  if (E * C == 0) return hipSuccess;
  if (bf16) {
    const int bm = grouped_gemm_bm_gate_up(true, C, d);
    if (bm == kSkinnyRows && d % 32 == 0)
      return launch_skinny<true>(buckets, wg, wu, h, kept, mtile_off, E, C, d, d_ff, wmap, s);
    if (bm == 320)
      return launch_bf16<320, 256, true>(buckets, wg, wu, h, kept, mtile_off, E, C, d, d_ff, wmap, s, sk, g, u);
    if (bm == 256)
      return launch_bf16<256, 256, true>(buckets, wg, wu, h, kept, mtile_off, E, C, d, d_ff, wmap, s, sk, g, u);
    if (d % 64 == 0)
      return launch_bf16<128, 256, true>(buckets, wg, wu, h, kept, mtile_off, E, C, d, d_ff, wmap, s);
    return launch_bf16<128, 128, true>(buckets, wg, wu, h, kept, mtile_off, E, C, d, d_ff, wmap, s);
  }
  const unsigned mtiles = static_cast<unsigned>(E * ceil_div(C, 64));
  gemm_f32_kernel<true><<<dim3(mtiles, static_cast<unsigned>(ceil_div(d_ff, 64))), dim3(256), 0, s>>>(
      static_cast<const float*>(buckets), static_cast<const float*>(wg), static_cast<const float*>(wu),
      static_cast<float*>(h), kept, mtile_off, E, C, d, d_ff, wmap);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const void* h, const int32_t* kept, const int32_t* mtile_off,
                            const void* wd, int E, int64_t C, int64_t d, int64_t d_ff, bool bf16,
                            void* y, hipStream_t s, const int32_t* wmap, const SplitK* sk, int bm) {
  if (E * C == 0) return hipSuccess;
  if (bf16) {
    const int tile = bm ? bm : grouped_gemm_bm(true, C);
    if (tile == kSkinnyRows && d_ff % 32 == 0)
      return launch_skinny<false>(h, wd, nullptr, y, kept, mtile_off, E, C, d_ff, d, wmap, s);
    if (tile == 320)
      return launch_bf16<320, 256, false>(h, wd, nullptr, y, kept, mtile_off, E, C, d_ff, d, wmap, s, sk);
    if (tile == 256)
      return launch_bf16<256, 256, false>(h, wd, nullptr, y, kept, mtile_off, E, C, d_ff, d, wmap, s, sk);
    if (d_ff % 64 == 0)
      return launch_bf16<128, 256, false>(h, wd, nullptr, y, kept, mtile_off, E, C, d_ff, d, wmap, s);
    return launch_bf16<128, 128, false>(h, wd, nullptr, y, kept, mtile_off, E, C, d_ff, d, wmap, s);
  }
  const unsigned mtiles = static_cast<unsigned>(E * ceil_div(C, 64));
  gemm_f32_kernel<false><<<dim3(mtiles, static_cast<unsigned>(ceil_div(d, 64))), dim3(256), 0, s>>>(
      static_cast<const float*>(h), static_cast<const float*>(wd), nullptr, static_cast<float*>(y), kept,
      mtile_off, E, C, d_ff, d, wmap);
  return hipGetLastError();
}

}  // namespace moe
