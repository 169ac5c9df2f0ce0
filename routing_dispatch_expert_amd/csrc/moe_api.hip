// Host side of the C ABI in include/moe.h: argument checks, workspace layout
// and the launch sequence of the MoE-layer hot path on the caller's stream.
// No device memory is allocated, no stream is synchronised and nothing is
// copied back to the host here.
#include "moe.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.h"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_stage_ev[2 * MOE_NUM_STAGES];
thread_local bool g_stage_ev_on = false;
thread_local bool g_stage_ran[MOE_NUM_STAGES] = {};

// Records the start (end = false) or end event of a stage when profiling is
// on; a stage that launches nothing (empty) records neither.
hipError_t stage_mark(int stage, bool end, hipStream_t s, bool empty = false) {
  if (!g_stage_ev_on) return hipSuccess;
  g_stage_ran[stage] = !empty;
  if (empty) return hipSuccess;
  return hipEventRecord(g_stage_ev[2 * stage + (end ? 1 : 0)], s);
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_err, sizeof(g_err), "%s: %s", what, hipGetErrorString(e));
  return MOE_ERR_HIP;
}

#define MOE_HIP_TRY(call, what)                      \
  do {                                               \
    hipError_t err_ = (call);                        \
    if (err_ != hipSuccess) return hip_fail(err_, what); \
  } while (0)

constexpr size_t kAlign = 256;
constexpr int kMaxE = 4096;
constexpr int kMaxK = 32;
constexpr int kMaxLimitRanks = 64;  // ranks of the rank-limited routing (one 64-bit mask)

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Sequential carving of one workspace block into 256-byte aligned arrays.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    off = align_up(off);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

int elem_bytes(moe_dtype_t dt) { return dt == MOE_DTYPE_BF16 ? 2 : 4; }

bool valid_dtype(int dt) { return dt == MOE_DTYPE_F32 || dt == MOE_DTYPE_BF16; }

int check_width(int64_t n, moe_dtype_t dt, const char* name) {
  const int64_t q = dt == MOE_DTYPE_BF16 ? 8 : 4;  // whole 16-byte words per row
  if (n % q) return fail(MOE_ERR_UNSUPPORTED, "%s=%lld must be a multiple of %lld", name,
                         static_cast<long long>(n), static_cast<long long>(q));
  return MOE_OK;
}

int capacity_of(int64_t T, int32_t E, int32_t k, float cf, int64_t* C) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%lld < 0", static_cast<long long>(T));
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E=%d < 1", E);
  if (k < 1) return fail(MOE_ERR_INVALID_ARG, "k=%d < 1", k);
  if (!std::isfinite(cf) || !(cf > 0.f)) return fail(MOE_ERR_INVALID_ARG, "cf must be finite and > 0");
  // ((cf * k) * T) / E in IEEE double, then ceil.
  const double c = std::ceil(static_cast<double>(cf) * static_cast<double>(k) * static_cast<double>(T) /
                             static_cast<double>(E));
  if (c > 9.0e15) return fail(MOE_ERR_UNSUPPORTED, "capacity too large");
  *C = static_cast<int64_t>(c);
  return MOE_OK;
}

// The grouped GEMM addresses one expert's rows and weights with 32-bit byte
// offsets: (C + 256) rows of max(d, d_ff) elements and d x d_ff weights.
int check_expert_extent(int64_t C, int64_t d, int64_t d_ff) {
  const int64_t lim = int64_t{1} << 31;
  if ((C + 256) * std::max(d, d_ff) * 4 >= lim || d * d_ff * 4 >= lim)
    return fail(MOE_ERR_UNSUPPORTED, "one expert's bucket or weight matrix exceeds 2^31 bytes");
  return MOE_OK;
}

// Rank limit of the routing: max_ranks = 0 (or >= P) is no limit; otherwise
// each token's experts lie on at most max_ranks of the P ranks.
int check_rank_limit(int32_t E, int32_t k, int32_t P, int32_t max_ranks) {
  if (P < 1 || E % P) return fail(MOE_ERR_INVALID_ARG, "P=%d must be >= 1 and divide E=%d", P, E);
  if (max_ranks < 0) return fail(MOE_ERR_INVALID_ARG, "max_ranks=%d must be >= 0", max_ranks);
  if (!moe::route_rank_limited(P, max_ranks)) return MOE_OK;
  if (P > kMaxLimitRanks) return fail(MOE_ERR_UNSUPPORTED, "rank-limited routing needs P <= %d", kMaxLimitRanks);
  if (static_cast<int64_t>(max_ranks) * (E / P) < k)
    return fail(MOE_ERR_INVALID_ARG, "max_ranks=%d ranks of %d experts hold fewer than k=%d", max_ranks, E / P, k);
  return MOE_OK;
}

// Checks shared by the layer entry points. Returns MOE_OK or an error status.
int check_layer_shape(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf, int32_t P,
                      int dtype, int64_t* C) {
  if (!valid_dtype(dtype)) return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (d < 1 || d_ff < 1) return fail(MOE_ERR_INVALID_ARG, "d and d_ff must be >= 1");
  int st = capacity_of(T, E, k, cf, C);
  if (st != MOE_OK) return st;
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "k=%d > E=%d", k, E);
  if (P < 1 || E % P) return fail(MOE_ERR_INVALID_ARG, "P=%d must be >= 1 and divide E=%d", P, E);
  const auto dt = static_cast<moe_dtype_t>(dtype);
  if ((st = check_width(d, dt, "d")) != MOE_OK) return st;
  if ((st = check_width(d_ff, dt, "d_ff")) != MOE_OK) return st;
  if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E=%d > %d", E, kMaxE);
  if (k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k=%d > %d", k, kMaxK);
  if (T * k >= (int64_t{1} << 31) || static_cast<int64_t>(E) * *C >= (int64_t{1} << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T*k and E*C must stay below 2^31");
  return check_expert_extent(*C, d, d_ff);
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const auto pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return an && bn && pa < pb + bn && pb < pa + an;
}

struct LayerPlan {
  float* logits;
  int32_t *idx, *slot, *tile_cnt, *tile_off, *routed, *kept, *send, *mtile, *mtile_gu, *src;
  float* w;
  int64_t* totals;
  void *buckets, *h, *y;
  moe::SplitK split;
  size_t bytes;
};

LayerPlan plan_layer(void* ws, int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, int64_t C,
                     int32_t P, int eb) {
  Carver c(ws);
  LayerPlan p;
  const int64_t nt = moe::ceil_div(T, moe::kTileTokens);
  const int S = moe::router_splits(T, d, E, eb == 2);
  p.logits = c.take<float>(static_cast<size_t>(S) * T * E);  // partial scores, S slices of d
  p.idx = c.take<int32_t>(static_cast<size_t>(T) * k);
  p.w = c.take<float>(static_cast<size_t>(T) * k);
  p.slot = c.take<int32_t>(static_cast<size_t>(T) * k);
  p.tile_cnt = c.take<int32_t>(static_cast<size_t>(nt) * E);
  p.tile_off = c.take<int32_t>(static_cast<size_t>(nt) * E);
  p.routed = c.take<int32_t>(E);
  p.kept = c.take<int32_t>(E);
  p.send = c.take<int32_t>(P);
  p.totals = c.take<int64_t>(MOE_NUM_TOTALS);
  p.mtile = c.take<int32_t>(static_cast<size_t>(E) + 1);
  p.mtile_gu = c.take<int32_t>(static_cast<size_t>(E) + 1);
  p.src = c.take<int32_t>(static_cast<size_t>(E) * C);
  p.buckets = c.take<char>(static_cast<size_t>(E) * C * d * eb);
  p.h = c.take<char>(static_cast<size_t>(E) * C * d_ff * eb);
  p.y = c.take<char>(static_cast<size_t>(E) * C * d * eb);
  p.split = moe::split_k_carve(c.take<char>(moe::split_k_bytes()));
  p.bytes = align_up(c.off);
  return p;
}

// Backward workspace: the forward plan (routing, buckets X, h, y) plus the
// recomputed g and u, the gradient rows and the transposed operands of the
// gradient GEMMs. Kp = C rounded up to 64: the row count the weight gradients
// contract over (rows past kept are zero in the transposed copies).
// The gradient GEMMs through the weights (dh = dy Wd, dX = [dg | du] [Wg ; Wu])
// read the weights K-major where the 256-row LDS-DMA kernel can: then no
// transposed weight copies are made.
bool backward_kmajor(bool bf16, int64_t C, int64_t d, int64_t F) {
  const int bm = moe::grouped_gemm_bm_contract_d(bf16, C, d);
  return bf16 && (bm == 256 || bm == 320) && d % 128 == 0 && F % 64 == 0;
}

struct BackPlan {
  LayerPlan f;
  void *g, *u, *dy, *dh, *dgu, *dX, *WdT, *WguT, *dyT, *hT, *dgT, *duT, *XT;
  float *dl, *rpart;
  int32_t *kfull_d, *kfull_f, *mtile_d, *mtile_f;
  int32_t *route_off, *lcopy, *ltok;  // routed copies listed per expert (router weight gradient)
  int64_t Kp;
  size_t bytes;
};

BackPlan plan_backward(void* ws, int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, int64_t C, int32_t P,
                       int eb) {
  BackPlan b;
  b.f = plan_layer(ws, T, d, d_ff, E, k, C, P, eb);
  Carver c(ws ? static_cast<char*>(ws) + b.f.bytes : nullptr);
  const size_t EC = static_cast<size_t>(E) * C;
  b.Kp = moe::ceil_div(C, 64) * 64;
  const size_t EKp = static_cast<size_t>(E) * b.Kp;
  b.g = c.take<char>(EC * d_ff * eb);
  b.u = c.take<char>(EC * d_ff * eb);
  b.dl = c.take<float>(static_cast<size_t>(T) * k);
  b.dy = c.take<char>(EC * d * eb);
  b.dh = c.take<char>(EC * d_ff * eb);
  b.dgu = c.take<char>(EC * 2 * d_ff * eb);
  b.dX = c.take<char>(EC * d * eb);
  const bool kmajor = backward_kmajor(eb == 2, C, d, d_ff);
  b.WdT = c.take<char>(kmajor ? 0 : static_cast<size_t>(E) * d_ff * d * eb);
  b.WguT = c.take<char>(kmajor ? 0 : static_cast<size_t>(E) * d * 2 * d_ff * eb);
  // bf16 weight gradients read the buckets K-major in place; fp32 contracts
  // over transposed copies
  const size_t tk = eb == 2 ? 0 : EKp;
  b.dyT = c.take<char>(tk * d * eb);
  b.hT = c.take<char>(tk * d_ff * eb);
  b.dgT = c.take<char>(tk * d_ff * eb);
  b.duT = c.take<char>(tk * d_ff * eb);
  b.XT = c.take<char>(tk * d * eb);
  b.kfull_d = c.take<int32_t>(E);
  b.kfull_f = c.take<int32_t>(E);
  b.mtile_d = c.take<int32_t>(static_cast<size_t>(E) + 1);
  b.mtile_f = c.take<int32_t>(static_cast<size_t>(E) + 1);
  b.rpart = c.take<float>(moe::router_wgrad_scratch_floats(T, k, E, d));
  b.route_off = c.take<int32_t>(static_cast<size_t>(E) + 1);
  b.lcopy = c.take<int32_t>(static_cast<size_t>(T) * k);
  b.ltok = c.take<int32_t>(static_cast<size_t>(T) * k);
  b.bytes = b.f.bytes + align_up(c.off);
  return b;
}

// Instances of replicated experts: E <= R <= 4096 (the scan's LDS), R*C < 2^31.
int check_replicas(int32_t E, int32_t R, int64_t C) {
  if (R < E || R > kMaxE) return fail(MOE_ERR_INVALID_ARG, "R=%d must be in [E=%d, %d]", R, E, kMaxE);
  if (static_cast<int64_t>(R) * C >= (int64_t{1} << 31)) return fail(MOE_ERR_UNSUPPORTED, "R*C must stay below 2^31");
  return MOE_OK;
}

// Replicated-layer workspace: routing as in the plain layer, the token-order
// rank of each copy within its expert, the instance maps, and the per-instance
// arrays (counts, row-tile map, buckets, h, y) for R instances.
struct ReplPlan {
  float *logits, *w;
  int32_t *idx, *qrank, *inst, *slot, *tile_cnt, *tile_off, *routed, *routed2, *kept1, *kept, *send, *send1,
      *mtile, *mtile_gu, *inst_off, *wmap, *place;
  int64_t *totals, *totals1;
  void *buckets, *h, *y;
  moe::SplitK split;
  size_t bytes;
};

ReplPlan plan_replicated(void* ws, int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, int64_t C, int32_t P,
                         int32_t R, int eb) {
  Carver c(ws);
  ReplPlan p;
  const int64_t nt = moe::ceil_div(T, moe::kTileTokens);
  const int S = moe::router_splits(T, d, E, eb == 2);
  const size_t Tk = static_cast<size_t>(T) * k;
  p.logits = c.take<float>(static_cast<size_t>(S) * T * E);
  p.idx = c.take<int32_t>(Tk);
  p.w = c.take<float>(Tk);
  p.qrank = c.take<int32_t>(Tk);
  p.inst = c.take<int32_t>(Tk);
  p.slot = c.take<int32_t>(Tk);
  p.tile_cnt = c.take<int32_t>(static_cast<size_t>(nt) * R);
  p.tile_off = c.take<int32_t>(static_cast<size_t>(nt) * R);
  p.routed = c.take<int32_t>(E);
  p.routed2 = c.take<int32_t>(R);
  p.kept1 = c.take<int32_t>(E);
  p.kept = c.take<int32_t>(R);
  p.send = c.take<int32_t>(P);
  p.send1 = c.take<int32_t>(P);
  p.totals = c.take<int64_t>(MOE_NUM_TOTALS);
  p.totals1 = c.take<int64_t>(MOE_NUM_TOTALS);
  p.mtile = c.take<int32_t>(static_cast<size_t>(R) + 1);
  p.mtile_gu = c.take<int32_t>(static_cast<size_t>(R) + 1);
  p.inst_off = c.take<int32_t>(static_cast<size_t>(E) + 1);
  p.wmap = c.take<int32_t>(R);
  p.place = c.take<int32_t>(R);
  p.buckets = c.take<char>(static_cast<size_t>(R) * C * d * eb);
  p.h = c.take<char>(static_cast<size_t>(R) * C * d_ff * eb);
  p.y = c.take<char>(static_cast<size_t>(R) * C * d * eb);
  p.split = moe::split_k_carve(c.take<char>(moe::split_k_bytes()));
  p.bytes = align_up(c.off);
  return p;
}

template <class T>
T* pick(T* user, T* fallback) {
  return user ? user : fallback;
}

// Argument checks of the permutation entry points: on the host, before any
// HIP call.
int check_permute(const void* x, const int32_t* topk_idx, int64_t T, int64_t d, int32_t E, int32_t k, int64_t C,
                  int32_t P, moe_dtype_t dtype, const void* buckets, const int32_t* slot,
                  const int32_t* routed_count, const int32_t* kept_count) {
  if (!valid_dtype(dtype)) return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E || C < 1)
    return fail(MOE_ERR_INVALID_ARG, "need T >= 0, d >= 1, 1 <= k <= E, C >= 1");
  if (P < 1 || E % P) return fail(MOE_ERR_INVALID_ARG, "P=%d must be >= 1 and divide E=%d", P, E);
  int st = check_width(d, dtype, "d");
  if (st != MOE_OK) return st;
  if (E > kMaxE || k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "E or k too large");
  if (T * k >= (int64_t{1} << 31) || E * C >= (int64_t{1} << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T*k and E*C must stay below 2^31");
  if (!x || !topk_idx || !buckets || !slot || !routed_count || !kept_count)
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  return MOE_OK;
}

// The permutation's launches over `scratch`, device memory of
// moe_permute_workspace_size() bytes, 256-byte aligned.
int run_permute(const void* x, const int32_t* topk_idx, int64_t T, int64_t d, int32_t E, int32_t k, int64_t C,
                int32_t P, moe_dtype_t dtype, void* buckets, int32_t* slot, int32_t* src, int32_t* routed_count,
                int32_t* kept_count, int32_t* send_count, int64_t* totals, void* scratch, hipStream_t s) {
  const int64_t nt = moe::ceil_div(T, moe::kTileTokens);
  Carver c(scratch);
  int32_t* tile_cnt = c.take<int32_t>(static_cast<size_t>(nt) * E);
  int32_t* tile_off = c.take<int32_t>(static_cast<size_t>(nt) * E);
  const int64_t row = d * elem_bytes(dtype);
  // ranks within each tile go to slot, then the slots (tile offset + rank) replace them
  // short tile histograms: the scan runs beside the slots and the row copies
  const bool one_pass = moe::slot_scatter_fits(T, k, E);
  MOE_HIP_TRY(moe::launch_tile_hist(topk_idx, T, k, E, tile_cnt, s, slot, one_pass && totals ? totals + 1 : nullptr),
              "tile histogram");
  if (one_pass) {
    MOE_HIP_TRY(moe::launch_slot_scatter(tile_cnt, E, C, P, row, k, T, tile_off, routed_count, kept_count,
                                         send_count, totals, 0, nullptr, 0, nullptr, nullptr, 0, x, topk_idx, slot,
                                         src, buckets, s),
                "slots and scatter");
    return MOE_OK;
  }
  MOE_HIP_TRY(moe::launch_scan(tile_cnt, nt, E, C, P, row, k, T, tile_off, routed_count, kept_count, send_count,
                               totals, 0, nullptr, src, s),
              "scan");
  MOE_HIP_TRY(moe::launch_slots_from_ranks(topk_idx, slot, tile_off, T, k, E, C, src, totals, s), "slots");
  MOE_HIP_TRY(moe::launch_scatter_rows(x, topk_idx, slot, T, k, C, row, buckets, s), "scatter");
  return MOE_OK;
}

// Scratch of moe_permute_static, for callers that cannot allocate: one copy
// per GPU (each device's module holds its own), kept until the process ends.
// Host code never uses the array's name as an address: static_scratch()
// asks the runtime for this device's copy once and keeps the pointer.
constexpr size_t kStaticScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = -1;
  MOE_HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MOE_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or size";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

int moe_set_stage_events(void* const* events, int n_events) {
  if (!events) {
    g_stage_ev_on = false;
    return MOE_OK;
  }
  if (n_events != 2 * MOE_NUM_STAGES)
    return fail(MOE_ERR_INVALID_ARG, "need %d events, got %d", 2 * MOE_NUM_STAGES, n_events);
  for (int i = 0; i < n_events; ++i) {
    if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "event %d is NULL", i);
    g_stage_ev[i] = static_cast<hipEvent_t>(events[i]);
  }
  g_stage_ev_on = true;
  return MOE_OK;
}

int moe_stage_ran(int32_t stage, int32_t* ran) {
  if (!ran) return fail(MOE_ERR_INVALID_ARG, "ran is NULL");
  if (stage < 0 || stage >= MOE_NUM_STAGES) return fail(MOE_ERR_INVALID_ARG, "no stage %d", stage);
  *ran = g_stage_ran[stage] ? 1 : 0;
  return MOE_OK;
}

int moe_capacity(int64_t T, int32_t E, int32_t k, float cf, int64_t* C_out) {
  if (!C_out) return fail(MOE_ERR_INVALID_ARG, "C_out is NULL");
  int64_t C;
  const int st = capacity_of(T, E, k, cf, &C);
  if (st == MOE_OK) *C_out = C;
  return st;
}

int moe_workspace_size(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf, int32_t P,
                       moe_dtype_t dtype, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  int64_t C;
  const int st = check_layer_shape(T, d, d_ff, E, k, cf, P, dtype, &C);
  if (st != MOE_OK) return st;
  *bytes = plan_layer(nullptr, T, d, d_ff, E, k, C, P, elem_bytes(dtype)).bytes;
  return MOE_OK;
}

int moe_layer_forward(const void* x, const void* W_router, const float* router_bias,
                      const void* W_gate, const void* W_up, const void* W_down, int64_t T,
                      int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf, int32_t P,
                      int32_t max_ranks, moe_dtype_t dtype, void* out, moe_stats_t* stats,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int64_t C;
  int st = check_layer_shape(T, d, d_ff, E, k, cf, P, dtype, &C);
  if (st != MOE_OK) return st;
  if ((st = check_rank_limit(E, k, P, max_ranks)) != MOE_OK) return st;
  if (!x || !W_router || !W_gate || !W_up || !W_down || !out)
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  const int eb = elem_bytes(dtype);
  if (overlaps(x, static_cast<size_t>(T * d * eb), out, static_cast<size_t>(T * d * eb)))
    return fail(MOE_ERR_INVALID_ARG, "out overlaps x");
  if (T == 0) return MOE_OK;
  const LayerPlan need = plan_layer(nullptr, T, d, d_ff, E, k, C, P, eb);
  if (!workspace || workspace_bytes < need.bytes || reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need.bytes);
  LayerPlan p = plan_layer(workspace, T, d, d_ff, E, k, C, P, eb);
  moe_stats_t none;
  std::memset(&none, 0, sizeof(none));
  const moe_stats_t& S = stats ? *stats : none;
  int32_t* idx = pick(S.topk_idx, p.idx);
  float* w = pick(S.topk_w, p.w);
  int32_t* slot = pick(S.slot, p.slot);
  int32_t* routed = pick(S.routed_count, p.routed);
  int32_t* kept = pick(S.kept_count, p.kept);
  int32_t* send = pick(S.send_count, p.send);
  int64_t* totals = pick(S.totals, p.totals);
  void* buckets = pick(S.buckets, p.buckets);
  int32_t* src = S.src;  // only built when asked for
  const bool bf16 = dtype == MOE_DTYPE_BF16;
  auto s = static_cast<hipStream_t>(stream);
  const int bm = moe::grouped_gemm_bm_down(bf16, C, d_ff);

  const int splits = moe::router_splits(T, d, E, bf16);
  MOE_HIP_TRY(stage_mark(MOE_STAGE_ROUTER, false, s), "event");
  MOE_HIP_TRY(moe::launch_router_logits(x, W_router, T, d, E, bf16, splits, p.logits, s), "router logits");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_ROUTER, true, s), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_ROUTE, false, s), "event");
  const bool fused_hist = moe::route_builds_histogram(k, E, T);
  const int64_t nt = moe::ceil_div(T, moe::kTileTokens);
  // short tile histograms: the scan runs beside the slots and the row copies,
  // which count fully dropped tokens into totals[1], zeroed by the histogram's kernel
  const bool one_pass = moe::slot_scatter_fits(T, k, E);
  int64_t* zero_t1 = one_pass ? totals + 1 : nullptr;
  // the tile histogram comes with each copy's rank within its tile, kept in slot
  MOE_HIP_TRY(moe::launch_route(p.logits, splits, router_bias, T, E, k, nullptr, idx, w,
                                fused_hist ? p.tile_cnt : nullptr, P, max_ranks, s, fused_hist ? slot : nullptr,
                                fused_hist ? zero_t1 : nullptr),
              "route");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_ROUTE, true, s), "event");
  // the scan also writes the counts, totals and both GEMMs' row-tile maps;
  // slots are the tile offsets plus the ranks
  const int bm_gu = moe::grouped_gemm_bm_gate_up(bf16, C, d);
  int32_t* mtile_gu = bm_gu != bm ? p.mtile_gu : nullptr;
  const bool slots_empty = fused_hist && one_pass;  // then the scatter's kernel does all of it
  MOE_HIP_TRY(stage_mark(MOE_STAGE_SLOTS, false, s, slots_empty), "event");
  if (!fused_hist) MOE_HIP_TRY(moe::launch_tile_hist(idx, T, k, E, p.tile_cnt, s, slot, zero_t1), "tile histogram");
  // the scan also clears the GEMMs' split-K arrival counters (each split tile's
  // last block leaves its counter at zero again, so GEMM 2 needs no clearing)
  moe::SplitK sk = p.split;
  sk.zeroed = sk.tick != nullptr;
  const int n_clear = sk.tick ? moe::kSplitUnits : 0;
  if (!one_pass) {
    MOE_HIP_TRY(moe::launch_scan(p.tile_cnt, nt, E, C, P, d * eb, k, T, p.tile_off, routed, kept, send, totals, bm,
                                 p.mtile, src, s, nullptr, bm_gu, mtile_gu, sk.tick, n_clear),
                "scan");
    MOE_HIP_TRY(moe::launch_slots_from_ranks(idx, slot, p.tile_off, T, k, E, C, src, totals, s), "slots");
  }
  MOE_HIP_TRY(stage_mark(MOE_STAGE_SLOTS, true, s, slots_empty), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_SCATTER, false, s), "event");
  if (one_pass)
    MOE_HIP_TRY(moe::launch_slot_scatter(p.tile_cnt, E, C, P, d * eb, k, T, p.tile_off, routed, kept, send, totals,
                                         bm, p.mtile, bm_gu, mtile_gu, sk.tick, n_clear, x, idx, slot, src, buckets,
                                         s),
                "slots and scatter");
  else
    MOE_HIP_TRY(moe::launch_scatter_rows(x, idx, slot, T, k, C, d * eb, buckets, s), "scatter");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_SCATTER, true, s), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_GATE_UP, false, s), "event");
  int32_t* map_gu = bm_gu != bm ? p.mtile_gu : p.mtile;
  void* h = p.h;
  const bool keep = S.g && S.u && S.h;
  if (keep) h = S.h;
  if (keep && moe::gate_up_keeps_gu(bf16, C, d)) {
    // g and u kept for the backward: the same GEMM also writes them rounded
    MOE_HIP_TRY(moe::launch_gemm_gate_up(buckets, kept, map_gu, W_gate, W_up, E, C, d, d_ff, bf16, h, s, nullptr,
                                         &sk, S.g, S.u),
                "grouped gemm (gate, up)");
  } else if (keep) {
    // elsewhere the two plain GEMMs and the SwiGLU product of their rounded
    // values, exactly as the backward recomputes them
    const int bmo = bf16 ? bm_gu : 0;
    MOE_HIP_TRY(moe::launch_gemm_down(buckets, kept, map_gu, W_gate, E, C, d_ff, d, bf16, S.g, s, nullptr, &sk, bmo),
                "grouped gemm (gate)");
    MOE_HIP_TRY(moe::launch_gemm_down(buckets, kept, map_gu, W_up, E, C, d_ff, d, bf16, S.u, s, nullptr, &sk, bmo),
                "grouped gemm (up)");
    MOE_HIP_TRY(moe::launch_swiglu_fwd(S.g, S.u, h, kept, E, C, d_ff, bf16, s), "swiglu");
  } else {
    MOE_HIP_TRY(moe::launch_gemm_gate_up(buckets, kept, map_gu, W_gate, W_up, E, C, d, d_ff, bf16, h, s, nullptr,
                                         &sk),
                "grouped gemm (gate, up)");
  }
  MOE_HIP_TRY(stage_mark(MOE_STAGE_GATE_UP, true, s), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_DOWN, false, s), "event");
  MOE_HIP_TRY(moe::launch_gemm_down(h, kept, p.mtile, W_down, E, C, d, d_ff, bf16, p.y, s, nullptr, &sk, bm),
              "grouped gemm (down)");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_DOWN, true, s), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_COMBINE, false, s), "event");
  MOE_HIP_TRY(moe::launch_combine(x, p.y, idx, w, slot, T, d, k, E, C, bf16, out, s), "combine");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_COMBINE, true, s), "event");
  return MOE_OK;
}

int moe_backward_workspace_size(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf, int32_t P,
                                moe_dtype_t dtype, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  int64_t C;
  const int st = check_layer_shape(T, d, d_ff, E, k, cf, P, dtype, &C);
  if (st != MOE_OK) return st;
  *bytes = plan_backward(nullptr, T, d, d_ff, E, k, C, P, elem_bytes(dtype)).bytes;
  return MOE_OK;
}

namespace {

// The backward; with `saved` (a kept forward state) the routing, buckets and
// activations are taken from it instead of being recomputed.
int layer_backward(const void* x, const void* W_router, const float* router_bias, const void* W_gate,
                   const void* W_up, const void* W_down, const void* dout, int64_t T, int64_t d, int64_t d_ff,
                   int32_t E, int32_t k, float cf, int32_t P, int32_t max_ranks, moe_dtype_t dtype,
                   const moe_stats_t* saved, void* dx, void* dW_router, float* d_bias, void* dW_gate, void* dW_up,
                   void* dW_down, void* workspace, size_t workspace_bytes, void* stream) {
  int64_t C;
  int st = check_layer_shape(T, d, d_ff, E, k, cf, P, dtype, &C);
  if (st != MOE_OK) return st;
  if ((st = check_rank_limit(E, k, P, max_ranks)) != MOE_OK) return st;
  if (!x || !W_router || !W_gate || !W_up || !W_down || !dout || !dx || !dW_router || !dW_gate || !dW_up ||
      !dW_down)
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  if (saved && (!saved->topk_idx || !saved->topk_w || !saved->buckets || !saved->g || !saved->u || !saved->h))
    return fail(MOE_ERR_INVALID_ARG, "saved state needs topk_idx, topk_w, buckets, g, u and h");
  const int eb = elem_bytes(dtype);
  const size_t row_bytes = static_cast<size_t>(T * d * eb);
  if (overlaps(dx, row_bytes, x, row_bytes) || overlaps(dx, row_bytes, dout, row_bytes))
    return fail(MOE_ERR_INVALID_ARG, "dx overlaps x or dout");
  const int64_t Kp = moe::ceil_div(C, 64) * 64;
  // the gradient GEMMs: rows d or d_ff contracting over Kp rows, and 2 d_ff
  if ((st = check_expert_extent(d, Kp, d_ff)) != MOE_OK || (st = check_expert_extent(d_ff, Kp, d)) != MOE_OK ||
      (st = check_expert_extent(C, d, 2 * d_ff)) != MOE_OK)
    return st;
  if (T == 0) return MOE_OK;
  const BackPlan need = plan_backward(nullptr, T, d, d_ff, E, k, C, P, eb);
  if (!workspace || workspace_bytes < need.bytes || reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need.bytes);
  BackPlan b = plan_backward(workspace, T, d, d_ff, E, k, C, P, eb);
  const LayerPlan& p = b.f;
  const bool bf16 = dtype == MOE_DTYPE_BF16;
  auto s = static_cast<hipStream_t>(stream);
  const int64_t nt = moe::ceil_div(T, moe::kTileTokens);
  const int bm = moe::grouped_gemm_bm(bf16, C);
  const int64_t F = d_ff;

  // 1. the forward again: routing, buckets X, g, u, h (y is not needed: the
  //    gate gradients come from dh and h, step 4); with a kept state only the
  //    counts, slots and per-expert copy lists, from its routing
  int32_t* idx = saved ? saved->topk_idx : p.idx;
  float* w = saved ? saved->topk_w : p.w;
  void* X = saved ? saved->buckets : p.buckets;
  void* g = saved ? saved->g : b.g;
  void* u = saved ? saved->u : b.u;
  void* h = saved ? saved->h : p.h;
  const int splits = moe::router_splits(T, d, E, bf16);
  const bool fused_hist = !saved && moe::route_builds_histogram(k, E, T);
  if (!saved) {
    MOE_HIP_TRY(moe::launch_router_logits(x, W_router, T, d, E, bf16, splits, p.logits, s), "router logits");
    MOE_HIP_TRY(moe::launch_route(p.logits, splits, router_bias, T, E, k, nullptr, idx, w,
                                  fused_hist ? p.tile_cnt : nullptr, P, max_ranks, s),
                "route");
  }
  if (!fused_hist) MOE_HIP_TRY(moe::launch_tile_hist(idx, T, k, E, p.tile_cnt, s), "tile histogram");
  // the scan also clears the split-K arrival counters once; each split tile's
  // last block leaves its counter at zero again for the next GEMM
  moe::SplitK split = p.split;
  split.zeroed = split.tick != nullptr;
  MOE_HIP_TRY(moe::launch_scan(p.tile_cnt, nt, E, C, P, d * eb, k, T, p.tile_off, p.routed, p.kept, p.send,
                               p.totals, bm, p.mtile, nullptr, s, nullptr, 0, nullptr, split.tick,
                               split.tick ? moe::kSplitUnits : 0),
              "scan");
  MOE_HIP_TRY(moe::launch_exclusive_scan(p.routed, E, b.route_off, s), "routed offsets");
  MOE_HIP_TRY(moe::launch_slots(idx, p.tile_off, T, k, E, C, p.slot, nullptr, p.totals, s, b.route_off, b.lcopy,
                                b.ltok),
              "slots");
  if (!saved) MOE_HIP_TRY(moe::launch_scatter_rows(x, idx, p.slot, T, k, C, d * eb, X, s), "scatter");
  // g = X Wg^T and u = X Wu^T (the plain row-tile GEMM: N = d_ff, K = d). GEMMs
  // that contract over d take the row-tile height of GEMM 1 (bm_d, map mtile_d_rows).
  const moe::SplitK* sk = &split;
  const int bm_d = moe::grouped_gemm_bm_contract_d(bf16, C, d);
  int32_t* mtile_d_rows = p.mtile;
  if (bm_d != bm) {
    MOE_HIP_TRY(moe::launch_mtile_map(p.kept, E, C, bm_d, p.mtile_gu, s), "tile map");
    mtile_d_rows = p.mtile_gu;
  }
  const int bmo_d = bf16 ? bm_d : 0;
  if (!saved && moe::gate_up_keeps_gu(bf16, C, d)) {  // GEMM 1 as the forward runs it, g and u kept
    MOE_HIP_TRY(moe::launch_gemm_gate_up(X, p.kept, mtile_d_rows, W_gate, W_up, E, C, d, F, bf16, h, s, nullptr, sk,
                                         g, u),
                "gemm g, u");
  } else if (!saved) {
    MOE_HIP_TRY(moe::launch_gemm_down(X, p.kept, mtile_d_rows, W_gate, E, C, F, d, bf16, g, s, nullptr, sk, bmo_d),
                "gemm g");
    MOE_HIP_TRY(moe::launch_gemm_down(X, p.kept, mtile_d_rows, W_up, E, C, F, d, bf16, u, s, nullptr, sk, bmo_d),
                "gemm u");
    MOE_HIP_TRY(moe::launch_swiglu_fwd(g, u, h, p.kept, E, C, F, bf16, s), "swiglu");
  }

  // 2. combine backward: dy = w dout on kept rows
  MOE_HIP_TRY(moe::launch_combine_bwd(dout, nullptr, idx, w, p.slot, T, d, k, C, bf16, b.dy, nullptr, s),
              "combine backward");
  // 3. dh = dy Wd; dg, du. 4. dX = [dg | du] [Wg ; Wu]. Either straight from the
  //    weights (K-major B: Wd is [d][d_ff] = [K][N], Wg and Wu are [d_ff][d]),
  //    or through transposed copies (B = Wd^T [E][d_ff][d], [Wg^T | Wu^T] [E][d][2 d_ff]).
  if (backward_kmajor(bf16, C, d, F)) {  // then bm_d is 256 or 320 and mtile_d_rows is its map
    MOE_HIP_TRY(moe::launch_gemm_kmajor_b(b.dy, p.kept, mtile_d_rows, W_down, nullptr, d, E, C, d, F, b.dh, s, sk,
                                          bm_d),
                "gemm dh");
    MOE_HIP_TRY(moe::launch_swiglu_bwd(b.dh, g, u, b.dgu, p.kept, E, C, F, bf16, s), "swiglu backward");
    MOE_HIP_TRY(moe::launch_gemm_kmajor_b(b.dgu, p.kept, mtile_d_rows, W_gate, W_up, F, E, C, 2 * F, d, b.dX, s, sk,
                                          bm_d),
                "gemm dX");
  } else {
    MOE_HIP_TRY(moe::launch_transpose(W_down, b.WdT, E, d, F, F, d, 0, d, nullptr, d * F, F * d, bf16, s),
                "transpose W_down");
    MOE_HIP_TRY(moe::launch_gemm_down(b.dy, p.kept, mtile_d_rows, b.WdT, E, C, F, d, bf16, b.dh, s, nullptr, sk,
                                      bmo_d),
                "gemm dh");
    MOE_HIP_TRY(moe::launch_swiglu_bwd(b.dh, g, u, b.dgu, p.kept, E, C, F, bf16, s), "swiglu backward");
    MOE_HIP_TRY(moe::launch_transpose(W_gate, b.WguT, E, F, d, d, 2 * F, 0, F, nullptr, F * d, d * 2 * F, bf16, s),
                "transpose W_gate");
    MOE_HIP_TRY(moe::launch_transpose(W_up, b.WguT, E, F, d, d, 2 * F, F, F, nullptr, F * d, d * 2 * F, bf16, s),
                "transpose W_up");
    MOE_HIP_TRY(moe::launch_gemm_down(b.dgu, p.kept, p.mtile, b.WguT, E, C, d, 2 * F, bf16, b.dX, s, nullptr, sk),
                "gemm dX");
  }
  //    the gate gradients: q_j = <dh_j, h_j> = w_j <dout, y_j>, dl_j = q_j - w_j sum_i q_i
  MOE_HIP_TRY(moe::launch_gate_grad(b.dh, h, idx, w, p.slot, T, F, k, C, bf16, b.dl, s), "gate gradients");
  // 5. router gradients, then dx = dout + the expert paths + the router path
  MOE_HIP_TRY(moe::launch_router_wgrad(x, idx, b.dl, T, k, E, d, bf16, b.rpart, dW_router, d_bias, s, p.routed,
                                       b.route_off, b.lcopy, b.ltok),
              "router wgrad");
  MOE_HIP_TRY(moe::launch_gather_dx(dout, b.dX, W_router, idx, b.dl, p.slot, T, d, k, C, bf16, dx, s),
              "gather dx");
  // 6. weight gradients over each expert's kept rows: dWd = dy^T h, dWg = dg^T X,
  //    dWu = du^T X. bf16: both operands read K-major straight from the
  //    buckets, each expert contracting over its own kept rows.
  if (bf16) {
    MOE_HIP_TRY(moe::launch_gemm_tn(b.dy, d, C * d, 0, h, C * F, p.kept, E, d, F, dW_down, s), "gemm dW_down");
    MOE_HIP_TRY(moe::launch_gemm_tn(b.dgu, 2 * F, C * 2 * F, 0, X, C * d, p.kept, E, F, d, dW_gate, s),
                "gemm dW_gate");
    MOE_HIP_TRY(moe::launch_gemm_tn(b.dgu, 2 * F, C * 2 * F, F, X, C * d, p.kept, E, F, d, dW_up, s),
                "gemm dW_up");
    return MOE_OK;
  }
  //    fp32: row-tile GEMMs of the transposed operands (M = d or d_ff rows
  //    for every expert, K = Kp)
  MOE_HIP_TRY(moe::launch_transpose(b.dy, b.dyT, E, C, d, d, b.Kp, 0, b.Kp, p.kept, C * d, d * b.Kp, bf16, s),
              "transpose dy");
  MOE_HIP_TRY(moe::launch_transpose(h, b.hT, E, C, F, F, b.Kp, 0, b.Kp, p.kept, C * F, F * b.Kp, bf16, s),
              "transpose h");
  MOE_HIP_TRY(moe::launch_transpose(b.dgu, b.dgT, E, C, F, 2 * F, b.Kp, 0, b.Kp, p.kept, C * 2 * F, F * b.Kp, bf16,
                                    s),
              "transpose dg");
  MOE_HIP_TRY(moe::launch_transpose(static_cast<char*>(b.dgu) + F * eb, b.duT, E, C, F, 2 * F, b.Kp, 0, b.Kp,
                                    p.kept, C * 2 * F, F * b.Kp, bf16, s),
              "transpose du");
  MOE_HIP_TRY(moe::launch_transpose(X, b.XT, E, C, d, d, b.Kp, 0, b.Kp, p.kept, C * d, d * b.Kp, bf16, s),
              "transpose X");
  MOE_HIP_TRY(moe::launch_fill_i32(b.kfull_d, E, static_cast<int32_t>(d), s), "fill");
  MOE_HIP_TRY(moe::launch_fill_i32(b.kfull_f, E, static_cast<int32_t>(F), s), "fill");
  MOE_HIP_TRY(moe::launch_mtile_map(b.kfull_d, E, d, moe::grouped_gemm_bm(bf16, d), b.mtile_d, s), "tile map");
  MOE_HIP_TRY(moe::launch_mtile_map(b.kfull_f, E, F, moe::grouped_gemm_bm(bf16, F), b.mtile_f, s), "tile map");
  MOE_HIP_TRY(moe::launch_gemm_down(b.dyT, b.kfull_d, b.mtile_d, b.hT, E, d, F, b.Kp, bf16, dW_down, s),
              "gemm dW_down");
  MOE_HIP_TRY(moe::launch_gemm_down(b.dgT, b.kfull_f, b.mtile_f, b.XT, E, F, d, b.Kp, bf16, dW_gate, s),
              "gemm dW_gate");
  MOE_HIP_TRY(moe::launch_gemm_down(b.duT, b.kfull_f, b.mtile_f, b.XT, E, F, d, b.Kp, bf16, dW_up, s),
              "gemm dW_up");
  return MOE_OK;
}

}  // namespace

int moe_layer_backward(const void* x, const void* W_router, const float* router_bias, const void* W_gate,
                       const void* W_up, const void* W_down, const void* dout, int64_t T, int64_t d, int64_t d_ff,
                       int32_t E, int32_t k, float cf, int32_t P, int32_t max_ranks, moe_dtype_t dtype, void* dx,
                       void* dW_router, float* d_bias, void* dW_gate, void* dW_up, void* dW_down,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return layer_backward(x, W_router, router_bias, W_gate, W_up, W_down, dout, T, d, d_ff, E, k, cf, P, max_ranks,
                        dtype, nullptr, dx, dW_router, d_bias, dW_gate, dW_up, dW_down, workspace, workspace_bytes,
                        stream);
}

int moe_layer_backward_saved(const void* x, const void* W_router, const float* router_bias, const void* W_gate,
                             const void* W_up, const void* W_down, const void* dout, int64_t T, int64_t d,
                             int64_t d_ff, int32_t E, int32_t k, float cf, int32_t P, int32_t max_ranks,
                             moe_dtype_t dtype, const moe_stats_t* saved, void* dx, void* dW_router, float* d_bias,
                             void* dW_gate, void* dW_up, void* dW_down, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!saved) return fail(MOE_ERR_INVALID_ARG, "saved is NULL");
  return layer_backward(x, W_router, router_bias, W_gate, W_up, W_down, dout, T, d, d_ff, E, k, cf, P, max_ranks,
                        dtype, saved, dx, dW_router, d_bias, dW_gate, dW_up, dW_down, workspace, workspace_bytes,
                        stream);
}

int moe_replica_plan(const int32_t* routed_count, int32_t E, int32_t extra, int32_t* replicas) {
  if (!routed_count || !replicas || E < 1 || extra < 0)
    return fail(MOE_ERR_INVALID_ARG, "need routed_count, replicas, E >= 1, extra >= 0");
  for (int e = 0; e < E; ++e) replicas[e] = 1;
  for (int n = 0; n < extra; ++n) {  // the highest load per replica gets the next one
    int best = 0;
    for (int e = 1; e < E; ++e)
      if (static_cast<int64_t>(routed_count[e]) * replicas[best] > static_cast<int64_t>(routed_count[best]) * replicas[e])
        best = e;
    ++replicas[best];
  }
  return MOE_OK;
}

int moe_replicated_workspace_size(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf, int32_t P,
                                  int32_t R, moe_dtype_t dtype, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  int64_t C;
  int st = check_layer_shape(T, d, d_ff, E, k, cf, P, dtype, &C);
  if (st != MOE_OK || (st = check_replicas(E, R, C)) != MOE_OK) return st;
  *bytes = plan_replicated(nullptr, T, d, d_ff, E, k, C, P, R, elem_bytes(dtype)).bytes;
  return MOE_OK;
}

int moe_layer_forward_replicated(const void* x, const void* W_router, const float* router_bias, const void* W_gate,
                                 const void* W_up, const void* W_down, int64_t T, int64_t d, int64_t d_ff, int32_t E,
                                 int32_t k, float cf, int32_t P, int32_t max_ranks, const int32_t* replicas,
                                 int32_t R, moe_dtype_t dtype, void* out, moe_stats_t* stats, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  int64_t C;
  int st = check_layer_shape(T, d, d_ff, E, k, cf, P, dtype, &C);
  if (st != MOE_OK) return st;
  if ((st = check_rank_limit(E, k, P, max_ranks)) != MOE_OK || (st = check_replicas(E, R, C)) != MOE_OK) return st;
  if (!x || !W_router || !W_gate || !W_up || !W_down || !out || !replicas)
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  const int eb = elem_bytes(dtype);
  if (overlaps(x, static_cast<size_t>(T * d * eb), out, static_cast<size_t>(T * d * eb)))
    return fail(MOE_ERR_INVALID_ARG, "out overlaps x");
  if (T == 0) return MOE_OK;
  const ReplPlan need = plan_replicated(nullptr, T, d, d_ff, E, k, C, P, R, eb);
  if (!workspace || workspace_bytes < need.bytes || reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need.bytes);
  ReplPlan p = plan_replicated(workspace, T, d, d_ff, E, k, C, P, R, eb);
  moe_stats_t none;
  std::memset(&none, 0, sizeof(none));
  const moe_stats_t& S = stats ? *stats : none;
  int32_t* idx = pick(S.topk_idx, p.idx);
  float* w = pick(S.topk_w, p.w);
  int32_t* slot = pick(S.slot, p.slot);
  int32_t* inst = pick(S.instance, p.inst);
  int32_t* routed = pick(S.routed_count, p.routed);
  int32_t* kept = pick(S.kept_count, p.kept);
  int32_t* send = pick(S.send_count, p.send);
  int64_t* totals = pick(S.totals, p.totals);
  void* buckets = pick(S.buckets, p.buckets);
  int32_t* src = S.src;
  const bool bf16 = dtype == MOE_DTYPE_BF16;
  auto s = static_cast<hipStream_t>(stream);
  const int64_t nt = moe::ceil_div(T, moe::kTileTokens);
  const int bm = moe::grouped_gemm_bm_down(bf16, C, d_ff);
  const int64_t no_cap = T * k;  // a capacity nothing exceeds

  // routing, then each copy's token-order rank among its expert's copies
  const int splits = moe::router_splits(T, d, E, bf16);
  const bool fused_hist = moe::route_builds_histogram(k, E, T);
  MOE_HIP_TRY(stage_mark(MOE_STAGE_ROUTER, false, s), "event");
  MOE_HIP_TRY(moe::launch_router_logits(x, W_router, T, d, E, bf16, splits, p.logits, s), "router logits");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_ROUTER, true, s), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_ROUTE, false, s), "event");
  MOE_HIP_TRY(moe::launch_route(p.logits, splits, router_bias, T, E, k, nullptr, idx, w,
                                fused_hist ? p.tile_cnt : nullptr, P, max_ranks, s),
              "route");
  if (!fused_hist) MOE_HIP_TRY(moe::launch_tile_hist(idx, T, k, E, p.tile_cnt, s), "tile histogram");
  MOE_HIP_TRY(moe::launch_scan(p.tile_cnt, nt, E, no_cap, P, d * eb, k, T, p.tile_off, routed, p.kept1, p.send1,
                               p.totals1, 0, nullptr, nullptr, s),
              "scan (experts)");
  MOE_HIP_TRY(moe::launch_slots(idx, p.tile_off, T, k, E, no_cap, p.qrank, nullptr, nullptr, s), "ranks");
  // instances, then the capacity-bounded permutation over them
  MOE_HIP_TRY(moe::launch_replica_layout(replicas, E, R, P, p.inst_off, p.wmap, p.place, s), "replica layout");
  MOE_HIP_TRY(moe::launch_instances(idx, p.qrank, replicas, p.inst_off, T * k, R, inst, s), "instances");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_ROUTE, true, s), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_SLOTS, false, s), "event");
  // the instances' slots: as in the plain layer, in one pass with the row
  // copies where the tile histogram is short enough. Their scan also writes
  // GEMM 1's row-tile map when its tiles differ from GEMM 2's, and clears the
  // GEMMs' split-K arrival counters (each split tile's last block leaves its
  // counter at zero again), so no GEMM needs a clearing launch.
  const int bm_gu = moe::grouped_gemm_bm_gate_up(bf16, C, d);
  int32_t* mtile_gu = bm_gu != bm ? p.mtile_gu : nullptr;
  moe::SplitK sk = p.split;
  sk.zeroed = sk.tick != nullptr;
  const int n_clear = sk.tick ? moe::kSplitUnits : 0;
  const bool one_pass = moe::slot_scatter_fits(T, k, R);
  MOE_HIP_TRY(moe::launch_tile_hist(inst, T, k, R, p.tile_cnt, s, one_pass ? slot : nullptr,
                                    one_pass ? totals + 1 : nullptr),
              "tile histogram (instances)");
  if (!one_pass) {
    MOE_HIP_TRY(moe::launch_scan(p.tile_cnt, nt, R, C, P, d * eb, k, T, p.tile_off, p.routed2, kept, send, totals,
                                 bm, p.mtile, src, s, p.place, bm_gu, mtile_gu, sk.tick, n_clear),
                "scan (instances)");
    MOE_HIP_TRY(moe::launch_slots(inst, p.tile_off, T, k, R, C, slot, src, totals, s), "slots");
  }
  MOE_HIP_TRY(stage_mark(MOE_STAGE_SLOTS, true, s), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_SCATTER, false, s), "event");
  if (one_pass)
    MOE_HIP_TRY(moe::launch_slot_scatter(p.tile_cnt, R, C, P, d * eb, k, T, p.tile_off, p.routed2, kept, send, totals,
                                         bm, p.mtile, bm_gu, mtile_gu, sk.tick, n_clear, x, inst, slot, src, buckets,
                                         s, p.place),
                "slots and scatter (instances)");
  else
    MOE_HIP_TRY(moe::launch_scatter_rows(x, inst, slot, T, k, C, d * eb, buckets, s), "scatter");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_SCATTER, true, s), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_GATE_UP, false, s), "event");
  MOE_HIP_TRY(moe::launch_gemm_gate_up(buckets, kept, mtile_gu ? mtile_gu : p.mtile, W_gate, W_up, R, C, d, d_ff,
                                       bf16, p.h, s, p.wmap, &sk),
              "grouped gemm (gate, up)");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_GATE_UP, true, s), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_DOWN, false, s), "event");
  MOE_HIP_TRY(moe::launch_gemm_down(p.h, kept, p.mtile, W_down, R, C, d, d_ff, bf16, p.y, s, p.wmap, &sk, bm),
              "grouped gemm (down)");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_DOWN, true, s), "event");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_COMBINE, false, s), "event");
  MOE_HIP_TRY(moe::launch_combine(x, p.y, inst, w, slot, T, d, k, R, C, bf16, out, s), "combine");
  MOE_HIP_TRY(stage_mark(MOE_STAGE_COMBINE, true, s), "event");
  return MOE_OK;
}

int moe_router_workspace_size(int64_t T, int64_t d, int32_t E, moe_dtype_t dtype, size_t* bytes) {
  if (!bytes || !valid_dtype(dtype) || T < 0 || d < 1 || E < 1)
    return fail(MOE_ERR_INVALID_ARG, "need bytes, a dtype, T >= 0, d >= 1, E >= 1");
  const int S = moe::router_splits(T, d, E, dtype == MOE_DTYPE_BF16);
  *bytes = align_up(static_cast<size_t>(S) * T * E * sizeof(float));
  return MOE_OK;
}

int moe_router(const void* x, const void* W_router, const float* router_bias, int64_t T, int64_t d,
               int32_t E, int32_t k, int32_t P, int32_t max_ranks, moe_dtype_t dtype,
               int32_t* topk_idx, float* topk_w, float* logits_out, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E)
    return fail(MOE_ERR_INVALID_ARG, "need T >= 0, d >= 1, 1 <= k <= E");
  int st = check_width(d, dtype, "d");
  if (st != MOE_OK) return st;
  if ((st = check_rank_limit(E, k, P, max_ranks)) != MOE_OK) return st;
  if (E > kMaxE || k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "E or k too large");
  if (T * k >= (int64_t{1} << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*k must stay below 2^31");
  if (!x || !W_router || !topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  if (T == 0) return MOE_OK;
  size_t need;
  moe_router_workspace_size(T, d, E, dtype, &need);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  auto s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == MOE_DTYPE_BF16;
  const int S = moe::router_splits(T, d, E, bf16);
  auto* part = static_cast<float*>(workspace);
  MOE_HIP_TRY(moe::launch_router_logits(x, W_router, T, d, E, bf16, S, part, s), "router logits");
  MOE_HIP_TRY(moe::launch_route(part, S, router_bias, T, E, k, logits_out, topk_idx, topk_w, nullptr, P,
                                max_ranks, s),
              "route");
  return MOE_OK;
}

int moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t P, int32_t max_ranks,
              int32_t* topk_idx, float* topk_w, void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "need T >= 0, 1 <= k <= E");
  const int st = check_rank_limit(E, k, P, max_ranks);
  if (st != MOE_OK) return st;
  if (E > kMaxE || k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "E or k too large");
  if (T * k >= (int64_t{1} << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*k must stay below 2^31");
  if (!logits || !topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  if (T == 0) return MOE_OK;
  MOE_HIP_TRY(moe::launch_route(logits, 1, nullptr, T, E, k, nullptr, topk_idx, topk_w, nullptr, P,
                                max_ranks, static_cast<hipStream_t>(stream)),
              "route");
  return MOE_OK;
}

int moe_permute_workspace_size(int64_t T, int32_t E, size_t* bytes) {
  if (!bytes || T < 0 || E < 1) return fail(MOE_ERR_INVALID_ARG, "need bytes, T >= 0, E >= 1");
  const size_t nt = static_cast<size_t>(moe::ceil_div(T, moe::kTileTokens));
  *bytes = 2 * align_up(nt * E * sizeof(int32_t));
  return MOE_OK;
}

int moe_permute(const void* x, const int32_t* topk_idx, int64_t T, int64_t d, int32_t E, int32_t k,
                int64_t C, int32_t P, moe_dtype_t dtype, void* buckets, int32_t* slot, int32_t* src,
                int32_t* routed_count, int32_t* kept_count, int32_t* send_count, int64_t* totals,
                void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_permute(x, topk_idx, T, d, E, k, C, P, dtype, buckets, slot, routed_count, kept_count);
  if (st != MOE_OK || T == 0) return st;
  size_t need;
  moe_permute_workspace_size(T, E, &need);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  return run_permute(x, topk_idx, T, d, E, k, C, P, dtype, buckets, slot, src, routed_count, kept_count, send_count,
                     totals, workspace, static_cast<hipStream_t>(stream));
}

int moe_permute_static(const void* x, const int32_t* topk_idx, int64_t T, int64_t d, int32_t E, int32_t k,
                       int64_t C, int32_t P, moe_dtype_t dtype, void* buckets, int32_t* slot, int32_t* src,
                       int32_t* routed_count, int32_t* kept_count, int32_t* send_count, int64_t* totals,
                       void* stream) {
  int st = check_permute(x, topk_idx, T, d, E, k, C, P, dtype, buckets, slot, routed_count, kept_count);
  if (st != MOE_OK || T == 0) return st;
  size_t need;
  moe_permute_workspace_size(T, E, &need);
  if (need > kStaticScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED, "T=%lld, E=%d need %zu bytes of scratch, more than the %zu of the static buffer",
                static_cast<long long>(T), E, need, kStaticScratchBytes);
  void* scr = nullptr;
  if ((st = static_scratch(&scr)) != MOE_OK) return st;
  return run_permute(x, topk_idx, T, d, E, k, C, P, dtype, buckets, slot, src, routed_count, kept_count, send_count,
                     totals, scr, static_cast<hipStream_t>(stream));
}

int moe_grouped_gemm_workspace_size(int32_t E, int64_t C, size_t* bytes) {
  if (!bytes || E < 1 || C < 1) return fail(MOE_ERR_INVALID_ARG, "need bytes, E >= 1, C >= 1");
  *bytes = 2 * align_up((static_cast<size_t>(E) + 1) * sizeof(int32_t)) + align_up(moe::split_k_bytes());
  return MOE_OK;
}

int moe_grouped_gemm(const void* buckets, const int32_t* kept_count, const void* W_gate,
                     const void* W_up, const void* W_down, int32_t E, int64_t C, int64_t d,
                     int64_t d_ff, moe_dtype_t dtype, void* h, void* y, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (E < 1 || C < 1 || d < 1 || d_ff < 1) return fail(MOE_ERR_INVALID_ARG, "need E, C, d, d_ff >= 1");
  int st = check_width(d, dtype, "d");
  if (st != MOE_OK || (st = check_width(d_ff, dtype, "d_ff")) != MOE_OK) return st;
  if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E=%d > %d", E, kMaxE);
  if (E * C >= (int64_t{1} << 31)) return fail(MOE_ERR_UNSUPPORTED, "E*C must stay below 2^31");
  if ((st = check_expert_extent(C, d, d_ff)) != MOE_OK) return st;
  if (!buckets || !kept_count || !W_gate || !W_up || !W_down || !h || !y)
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  size_t need;
  moe_grouped_gemm_workspace_size(E, C, &need);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  auto s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == MOE_DTYPE_BF16;
  const size_t map_bytes = align_up((static_cast<size_t>(E) + 1) * sizeof(int32_t));
  auto* mtile = static_cast<int32_t*>(workspace);
  auto* mtile_gu = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + map_bytes);
  const moe::SplitK sk = moe::split_k_carve(static_cast<char*>(workspace) + 2 * map_bytes);
  const int bm = moe::grouped_gemm_bm_down(bf16, C, d_ff);
  MOE_HIP_TRY(moe::launch_mtile_map(kept_count, E, C, bm, mtile, s), "tile map");
  MOE_HIP_TRY(moe::launch_mtile_map(kept_count, E, C, moe::grouped_gemm_bm_gate_up(bf16, C, d), mtile_gu, s), "tile map");
  MOE_HIP_TRY(moe::launch_gemm_gate_up(buckets, kept_count, mtile_gu, W_gate, W_up, E, C, d, d_ff, bf16, h, s,
                                       nullptr, &sk),
              "grouped gemm (gate, up)");
  MOE_HIP_TRY(moe::launch_gemm_down(h, kept_count, mtile, W_down, E, C, d, d_ff, bf16, y, s, nullptr, &sk, bm),
              "grouped gemm (down)");
  return MOE_OK;
}

int moe_combine(const void* x, const void* y, const int32_t* topk_idx, const float* topk_w,
                const int32_t* slot, int64_t T, int64_t d, int32_t E, int32_t k, int64_t C,
                moe_dtype_t dtype, void* out, void* stream) {
  if (!valid_dtype(dtype)) return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E || C < 1)
    return fail(MOE_ERR_INVALID_ARG, "need T >= 0, d >= 1, 1 <= k <= E, C >= 1");
  const int st = check_width(d, dtype, "d");
  if (st != MOE_OK) return st;
  if (k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k=%d > %d", k, kMaxK);
  if (!x || !y || !topk_idx || !topk_w || !slot || !out)
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  const size_t row = static_cast<size_t>(d) * elem_bytes(dtype);
  if (overlaps(x, T * row, out, T * row)) return fail(MOE_ERR_INVALID_ARG, "out overlaps x");
  if (T == 0) return MOE_OK;
  MOE_HIP_TRY(moe::launch_combine(x, y, topk_idx, topk_w, slot, T, d, k, E, C, dtype == MOE_DTYPE_BF16, out,
                                  static_cast<hipStream_t>(stream)),
              "combine");
  return MOE_OK;
}

}  // extern "C"
