// C ABI of libmoe (declared in include/moe.h): host-side validation, the
// static workspace plan and launch sequencing.  No allocation, no
// synchronisation, no device reads on the host.
#include <math.h>
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "kernels_f8f8.hpp"
#include "moe.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";
thread_local void* const* g_events = nullptr;
thread_local int g_nevents = 0;

// records the i-th timing event of moe_forward when the hook is armed
void mark(int i, int n_launches, hipStream_t s) {
  if (g_events && g_nevents > n_launches) (void)hipEventRecord((hipEvent_t)g_events[i], s);
}

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

constexpr int kSingleMaxT = 256;   // T up to which routing runs as split router + route_small
static_assert(kSingleMaxT * kMaxK <= kSmallMaxPairs, "every small-T forward must fit the small route's pair buffers");
constexpr int kStreamMaxT = 64;    // T up to which the expert GEMMs use the streaming kernels
constexpr int kA8StreamMaxT = 32;  // the same with FP8 activations
constexpr int64_t kMaxT = 1 << 20;
// The 256-row tiled kernels (ffn_tiled256.hip, eight waves) and when the plan takes them.  By
// default: the bf16 gate/up GEMM of a layer with a long K (d >= 4096) whose experts average at
// least 128 rows, on the many-token route path; its down GEMM keeps 128-row items (a second
// tile map).  Measured on the DeepSeek-V3-shaped layer (d = 7168), one GPU: gate/up T=16384
// 9.58 -> 9.12 ms, T=4096 3.59 -> 3.45 ms; down T=16384 4.56 -> 4.88 ms, T=4096 1.69 -> 1.91 ms
// (K = F = 2048 is too short for the deeper ring to pay); and with d = 2048 gate/up loses too
// (OLMoE T=4096 365 -> 402 us, DeepSeek-V2-Lite T=8192 800 -> 825 us).  The environment variable
// MOE_ROWS256_MIN_AVG, read at every plan, overrides the rule for both GEMMs: a positive n takes
// the 256-row kernels wherever experts average at least n rows, 0 never (the GPU tests use both
// to check the kernels against each other bit for bit).
constexpr int64_t kRows256Default = -1;
int64_t rows256_min_avg() {
  const char* v = getenv("MOE_ROWS256_MIN_AVG");
  if (!v || !*v) return kRows256Default;
  char* end = nullptr;
  const long long n = strtoll(v, &end, 10);
  if (!end || *end != 0 || n < 0) return kRows256Default;
  return (int64_t)(n < (1 << 30) ? n : (1 << 30));  // 0: never
}

struct Plan {
  int T, d, E, k, F, S, FS, act, wdt, score, renorm, tiled;
  int G, GM;  // expert groups, groups a token may pick from (0: no group limit)
  float gscale;
  int64_t cap;  // -1: dropless
  int64_t R;
  bool single;
  int KS, kchunk;
  int rt, n_rt, rpb, n_rb;
  int mode, bm;
  int bm_dn;  // rows per item of the down GEMM (bm unless the gate/up GEMM takes 256-row items alone)
  bool wstream;  // tiled kernels stream the weights non-temporally
  bool rowskip_gu, rowskip_dn;  // tiled kernels skip the idle row tiles of partly filled items
  int64_t items_max, items_max_dn;
  int sh_items, sh_items_dn;
  size_t o_part, o_arrived, o_hist, o_counts, o_off, o_rowtok, o_slot, o_items, o_nitems, o_items_dn, o_nitems_dn, o_h,
      o_hsh, o_y, o_ysh, o_xq, o_xs, o_hq, o_hs, o_hshq, o_hshs, total;
  bool a8;  // FP8 activations on the FP8 MFMA (MOE_FP8_E4M3_A8)
};

bool fp8_weights(int wdt) { return wdt == MOE_FP8_E4M3 || wdt == MOE_FP8_E4M3_A8; }

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

moe_status make_plan(const moe_cfg* c, Plan* p) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->T < 0 || c->T > kMaxT) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, %lld]", c->T, (long long)kMaxT);
  if (c->E < 1 || c->E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E=%d outside [1, 256]", c->E);
  if (c->k < 1 || c->k > kMaxK || c->k > c->E) return fail(MOE_ERR_UNSUPPORTED, "k=%d outside [1, min(E, 8)]", c->k);
  if (c->d < 128 || c->d % 128 || c->d > 65536) return fail(MOE_ERR_UNSUPPORTED, "d=%d is not a multiple of 128 in [128, 65536]", c->d);
  if (c->ffn < 128 || c->ffn % 128 || c->ffn > 65536)
    return fail(MOE_ERR_UNSUPPORTED, "ffn=%d is not a multiple of 128 in [128, 65536]", c->ffn);
  if (c->n_shared < 0 || c->n_shared > 8) return fail(MOE_ERR_UNSUPPORTED, "n_shared=%d outside [0, 8]", c->n_shared);
  if (c->n_shared > 0 && (c->ffn_shared < 128 || c->ffn_shared % 128 || c->ffn_shared > 65536))
    return fail(MOE_ERR_UNSUPPORTED, "ffn_shared=%d is not a multiple of 128 in [128, 65536]", c->ffn_shared);
  if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "act_dtype=%d is not MOE_F32 or MOE_BF16", c->act_dtype);
  if (c->expert_dtype != MOE_F32 && c->expert_dtype != MOE_BF16 && c->expert_dtype != MOE_INT4_G128 &&
      !fp8_weights(c->expert_dtype))
    return fail(MOE_ERR_INVALID_ARG, "expert_dtype=%d is not a moe_dtype", c->expert_dtype);
  const bool quant = c->expert_dtype == MOE_INT4_G128 || fp8_weights(c->expert_dtype);
  if (!(c->expert_dtype == c->act_dtype || (quant && c->act_dtype == MOE_BF16)))
    return fail(MOE_ERR_UNSUPPORTED, "expert_dtype=%d with act_dtype=%d", c->expert_dtype, c->act_dtype);
  if (c->score != MOE_SCORE_SOFTMAX && c->score != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "score=%d is not a moe_score", c->score);
  if (c->renorm != 0 && c->renorm != 1) return fail(MOE_ERR_INVALID_ARG, "renorm=%d is not 0 or 1", c->renorm);
  if (!isfinite(c->gate_scale)) return fail(MOE_ERR_INVALID_ARG, "gate_scale is not finite");
  if (c->weight_layout != MOE_LAYOUT_ROWS && c->weight_layout != MOE_LAYOUT_TILED)
    return fail(MOE_ERR_INVALID_ARG, "weight_layout=%d is not a moe_layout", c->weight_layout);
  {
    // every expert matrix must stay below 2 GiB (32-bit byte offsets inside one matrix)
    const int64_t nmax = c->ffn > (c->n_shared ? c->ffn_shared : 0) ? c->ffn : c->ffn_shared;
    const int64_t bytes = nmax * c->d * (c->expert_dtype == MOE_F32 ? 4 : 2);
    if (bytes >= ((int64_t)1 << 31))
      return fail(MOE_ERR_UNSUPPORTED, "an expert matrix of %lld bytes exceeds 2 GiB", (long long)bytes);
  }
  if (!(c->n_groups == 0 && c->topk_groups == 0)) {
    if (c->n_groups < 1 || c->n_groups > 64 || c->E % c->n_groups)
      return fail(MOE_ERR_UNSUPPORTED, "n_groups=%d: need 0, or 1..64 dividing E=%d", c->n_groups, c->E);
    if (c->topk_groups < 1 || c->topk_groups > c->n_groups || c->k > c->topk_groups * (c->E / c->n_groups))
      return fail(MOE_ERR_INVALID_ARG, "topk_groups=%d: need 1..n_groups with k <= topk_groups * E / n_groups",
                  c->topk_groups);
  }
  const bool dropless = c->cap_num == 0 && c->cap_den == 0;
  if (!dropless && (c->cap_den <= 0 || c->cap_num < 0))
    return fail(MOE_ERR_INVALID_ARG, "capacity %d/%d: need 0/0 or num >= 0, den > 0", c->cap_num, c->cap_den);

  Plan& q = *p;
  q.T = c->T;
  q.d = c->d;
  q.E = c->E;
  q.k = c->k;
  q.F = c->ffn;
  q.S = c->n_shared;
  q.FS = c->n_shared ? c->ffn_shared : 0;
  q.act = c->act_dtype;
  q.wdt = c->expert_dtype;
  q.G = c->n_groups;
  q.GM = c->topk_groups;
  q.score = c->score;
  q.renorm = c->renorm;
  q.gscale = c->gate_scale;
  q.tiled = c->weight_layout == MOE_LAYOUT_TILED;
  const int64_t pairs = (int64_t)q.T * q.k;
  if (dropless) {
    q.cap = -1;
    q.R = pairs;
  } else {
    const int64_t num = (int64_t)c->cap_num * q.T * q.k, den = (int64_t)c->cap_den * q.E;
    q.cap = (num + den - 1) / den;
    if (q.cap > pairs) q.cap = pairs;  // a larger cap keeps everything; also keeps it in int range
    q.R = q.cap * q.E < pairs ? q.cap * q.E : pairs;
  }
  q.single = q.T <= kSingleMaxT;
  // K split of the small-T router: each block of the route launch reads at most kSmallPartials
  // partial logits
  if (q.single && q.T > 0) {
    int64_t ks = kSmallPartials / ((int64_t)route_small_tpb(q.T) * q.E);
    const int64_t ksmax = q.d / 128;
    ks = ks < 1 ? 1 : (ks > ksmax ? ksmax : ks);
    const int64_t steps = q.d / 128;
    const int64_t per = (steps + ks - 1) / ks;
    q.kchunk = (int)(per * 128);
    q.KS = (int)((q.d + q.kchunk - 1) / q.kchunk);
  } else {
    q.KS = 0;
    q.kchunk = q.d;
  }
  // router tokens per tile: 16 (router_fused_kernel), or 64 for bf16 with more than 128 experts
  // from T = 8192 on (router_wide_kernel: the waves split the experts, so the 3.7 MB DeepSeek-V3
  // router weight is read once per 64 tokens; measured there, T=16384 646 -> 219 us, T=8192
  // 325 -> 206 us, but with fewer than 128 blocks it loses: T=4096 164 -> 200 us)
  q.rt = (q.E > 128 && q.act == MOE_BF16 && q.T >= 8192) ? 64 : 16;
  q.n_rt = (q.T + q.rt - 1) / q.rt;
  // at most kMaxRouteBlocks router (and permute) blocks, each over rpb consecutive router tiles:
  // every permute block sums the histograms of the blocks before it, so that work grows with the
  // square of the block count (512 blocks: at most 512 KB of reads per block at E = 256)
  q.rpb = (q.n_rt + kMaxRouteBlocks - 1) / kMaxRouteBlocks;
  if (q.rpb < 1) q.rpb = 1;
  q.n_rb = (q.n_rt + q.rpb - 1) / q.rpb;
  q.a8 = q.wdt == MOE_FP8_E4M3_A8;
  // FP8 activations: the tiled FP8 MFMA kernels, or up to kA8StreamMaxT tokens the streaming FP8
  // kernels on the codes held as bf16 (exact), with the row scales in their epilogues
  q.mode = q.a8 ? (q.T <= kA8StreamMaxT ? 0 : 1) : ((q.act == MOE_F32 || q.T <= kStreamMaxT) ? 0 : 1);
  // streaming kernels take items of 16 rows (T <= 16: an expert gets each token at most once; or
  // at most 8 pairs per expert on average, where splitting a hot expert costs less than the
  // registers of 32-row items: measured on OLMoE T=64, 170 -> 161 us) or 32 rows; above 32 a hot
  // expert is split into two items (its weights are read twice), which costs less than the
  // registers (occupancy) of 64-row items
  // tiled bf16 kernels: 256-row items per the rule above rows256_min_avg()
  bool gu256 = false, dn256 = false;
  if (q.wdt == MOE_BF16 && q.mode == 1) {
    const int64_t env = rows256_min_avg(), tk = (int64_t)q.T * q.k;
    if (env > 0) gu256 = dn256 = tk >= env * q.E;
    else if (env < 0) gu256 = !q.single && q.d >= 4096 && tk >= (int64_t)kPrefillRows * q.E;
  }
  q.bm = q.mode == 1 ? (gu256 ? 2 * kPrefillRows : kPrefillRows)
                     : ((q.T <= 16 || (int64_t)q.T * q.k <= 8 * (int64_t)q.E) ? 16 : 32);
  q.bm_dn = q.mode == 1 ? (dn256 ? 2 * kPrefillRows : kPrefillRows) : q.bm;
  // tiled mode with at most 32 rows per expert on average: an expert's weights are read by one
  // row tile (measured: DeepSeek-V3 T=256 2.81 -> 2.61 ms; with several row tiles per expert the
  // L2 reuse they lose costs far more, e.g. OLMoE T=4096 gate/up 313 -> 401 us)
  q.wstream = q.mode == 1 && (int64_t)q.T * q.k <= 32 * (int64_t)q.E;
  // tiled mode: an expert's last item usually holds fewer than 128 rows, and its idle 32-row tiles
  // can be skipped.  That tile then runs ahead of the expert's other tiles over the same weight
  // slab and can turn their L2 hits into misses; measured, skipping pays with INT4 weights (a
  // quarter of the bytes; Qwen3 INT4 T=4096 gate/up 288 -> 261 us) and with bf16 weights when
  // experts average at least two items and the slab's K is at most 4096 (OLMoE T=4096 gate/up
  // 315 -> 305 us), and costs 3% on DeepSeek-V3 (K = 7168, or T=4096 at 128 rows per expert).
  // With streamed weights (one row tile per expert) there is no reuse to lose (OLMoE T=256
  // 223 -> 208 us), unless shared experts follow: their full tiles, cut into the last XCD chunks
  // at the weight of the cheap routed ones, then finish last (DeepSeek-V2-Lite T=256 gate/up
  // 137 -> 152 us)
  {
    const bool many = (int64_t)q.T * q.k >= 2 * (int64_t)kPrefillRows * q.E;
    const bool lone = q.wstream && q.S == 0;
    q.rowskip_gu = q.wdt == MOE_INT4_G128 || lone || (many && q.d <= 4096);
    q.rowskip_dn = q.wdt == MOE_INT4_G128 || lone || (many && q.F <= 4096);
    // 256-row items: skip where experts average fewer than two items, so that few weight slabs
    // are shared between items (DeepSeek-V3 T=4096 gate/up 3.55-3.59 -> 3.36-3.39 ms); at two or
    // more the same loss of L2 reuse as above (DeepSeek-V3 T=16384 gate/up: 22% more bytes
    // fetched beyond L2, time unchanged)
    const bool few256 = (int64_t)q.T * q.k < 2 * (int64_t)(2 * kPrefillRows) * q.E;
    if (gu256) q.rowskip_gu = few256;
    if (dn256) q.rowskip_dn = few256;
  }
  q.items_max = q.R / q.bm + (q.R < q.E ? q.R : q.E);
  q.sh_items = q.S > 0 ? (q.T + q.bm - 1) / q.bm : 0;
  q.items_max_dn = q.R / q.bm_dn + (q.R < q.E ? q.R : q.E);
  q.sh_items_dn = q.S > 0 ? (q.T + q.bm_dn - 1) / q.bm_dn : 0;

  const size_t es = q.act == MOE_F32 ? 4 : 2;
  const size_t cs = q.mode == 0 ? 2 : 1;  // bytes per E4M3 code: bf16 values for the streaming kernels
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  q.o_part = take(q.single ? (size_t)q.KS * q.T * q.E * 4 : 0);
  q.o_arrived = take(4);
  q.o_hist = take(q.single ? 0 : (size_t)q.n_rb * q.E * 4);
  q.o_counts = take((size_t)q.E * 4);
  q.o_off = take((size_t)(q.E + 1) * 4);
  q.o_rowtok = take((size_t)q.R * 4);
  q.o_slot = take((size_t)pairs * 4);
  q.o_items = take((size_t)q.items_max * 16);
  q.o_nitems = take(4);
  q.o_items_dn = q.bm_dn != q.bm ? take((size_t)q.items_max_dn * 16) : q.o_items;
  q.o_nitems_dn = q.bm_dn != q.bm ? take(4) : q.o_nitems;
  q.o_h = take((size_t)q.R * q.F * es);
  q.o_hsh = take((size_t)q.T * q.S * q.FS * es);
  q.o_y = take((size_t)q.R * q.d * es);
  q.o_ysh = take(q.S ? (size_t)q.T * q.d * es : 0);
  q.o_xq = take(q.a8 ? (size_t)q.T * q.d * cs : 0);
  q.o_xs = take(q.a8 ? (size_t)q.T * 4 : 0);
  q.o_hq = take(q.a8 ? (size_t)q.R * q.F * cs : 0);
  q.o_hs = take(q.a8 ? (size_t)q.R * 4 : 0);
  q.o_hshq = take(q.a8 && q.S ? (size_t)q.T * q.S * q.FS * cs : 0);
  q.o_hshs = take(q.a8 && q.S ? (size_t)q.T * 4 : 0);
  q.total = o;
  return MOE_OK;
}

template <typename T> T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3) == 0; }
bool al2(const void* p) { return ((uintptr_t)p & 1) == 0; }

moe_status check_ws(const Plan& p, void* ws, size_t ws_bytes) {
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (!al16(ws)) return fail(MOE_ERR_WORKSPACE, "workspace is not 16-byte aligned");
  if (ws_bytes < p.total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, p.total);
  return MOE_OK;
}

moe_status hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A single token: the down projection and the combine run as one launch
// (down_combine_one_kernel), so a forward is four launches.  Measured (graph replays, one GPU):
// Qwen3 INT4-shaped T=1 37.4 -> 34.8 us, OLMoE-shaped FP8 T=1 35.9 -> 33.0 us, bf16 OLMoE-shaped
// T=1 41.8 -> 40.3 us, DeepSeek-V2-Lite-shaped T=1 51.9 -> 50.3 us, DeepSeek-V3-shaped T=1
// 154.2 -> 150.4 us (means of two rounds).
bool one_token(const Plan& p) { return p.T == 1 && p.mode == 0 && !p.a8; }

// the down GEMM's arguments: its own tile map when its items differ from the gate/up GEMM's
FfnArgs down_args(const Plan& p, void* ws, FfnArgs a) {
  a.items = at<int4>(ws, p.o_items_dn);
  a.n_items = at<int32_t>(ws, p.o_nitems_dn);
  a.items_max = (int)p.items_max_dn;
  a.sh_items = p.sh_items_dn;
  a.bm = p.bm_dn;
  return a;
}

// FP8 activations: E4M3 codes and row scales of x ahead of the gate/up GEMM, and of the routed
// and shared h ahead of the down GEMM (every one of the R routed rows: rows past the kept count
// hold stale values whose codes no tile reads)
A8Args a8_args(const Plan& p, void* ws) {
  A8Args q;
  q.xq = at<uint8_t>(ws, p.o_xq);
  q.xs = at<float>(ws, p.o_xs);
  q.hq = at<uint8_t>(ws, p.o_hq);
  q.hs = at<float>(ws, p.o_hs);
  q.hshq = p.S ? at<uint8_t>(ws, p.o_hshq) : nullptr;
  q.hshs = p.S ? at<float>(ws, p.o_hshs) : nullptr;
  return q;
}
// the gate/up GEMM (and with FP8 activations the quantisation of x before it)
moe_status enqueue_gateup(const Plan& p, void* ws, const FfnArgs& a, hipStream_t s) {
  if (!p.a8) return hip_ok(launch_ffn_gateup(p.mode, p.act, p.wdt, a, s), "gate/up GEMM");
  const A8Args q = a8_args(p, ws);
  const bool str = p.mode == 0;
  moe_status st = hip_ok(launch_quant_rows(a.x, q.xq, q.xs, p.T, p.d, nullptr, nullptr, nullptr, 0, 0, str, s),
                         "activation quantisation");
  if (st) return st;
  if (!str) return hip_ok(launch_ffn_a8(true, a, q, s), "gate/up GEMM");
  FfnArgs b = a;
  b.x = q.xq;  // the x codes as bf16
  return hip_ok(launch_ffn_a8_stream(true, b, q, s), "gate/up GEMM");
}
// the down GEMM (a: its own tile map; with FP8 activations the quantisation of h before it)
moe_status enqueue_down(const Plan& p, void* ws, const FfnArgs& a, hipStream_t s) {
  if (!p.a8) return hip_ok(launch_ffn_down(p.mode, p.act, p.wdt, a, s), "down GEMM");
  const A8Args q = a8_args(p, ws);
  const bool str = p.mode == 0;
  moe_status st = hip_ok(launch_quant_rows(a.h, q.hq, q.hs, (int)p.R, p.F, p.S ? a.hsh : nullptr,
                                           q.hshq, q.hshs, p.T, p.S * p.FS, str, s),
                         "intermediate quantisation");
  if (st) return st;
  if (!str) return hip_ok(launch_ffn_a8(false, a, q, s), "down GEMM");
  FfnArgs b = a;
  b.h = q.hq;  // the h codes as bf16
  b.hsh = q.hshq;
  return hip_ok(launch_ffn_a8_stream(false, b, q, s), "down GEMM");
}

// the expert GEMMs and the combine of moe_forward / moe_forward_with_routes
// (timing marks 3.. for moe_forward only: `timed`)
moe_status enqueue_experts_and_combine(const Plan& p, void* ws, const FfnArgs& a, const int32_t* topk_idx,
                                       const int32_t* slot, const float* topk_w, const void* ysh, void* out,
                                       hipStream_t s, bool timed) {
  const int nl = timed ? (one_token(p) ? 4 : 5) : 1 << 30;  // an impossible count records nothing
  moe_status st;
  if ((st = enqueue_gateup(p, ws, a, s))) return st;
  mark(3, nl, s);
  if (one_token(p)) {
    st = hip_ok(launch_down_combine_one(p.wdt, a, topk_idx, slot, topk_w, out, p.k, s), "down GEMM + combine");
    mark(4, nl, s);
    return st;
  }
  if ((st = enqueue_down(p, ws, down_args(p, ws, a), s))) return st;
  mark(4, nl, s);
  st = hip_ok(launch_combine(p.act, a.y, slot, topk_w, ysh, out, p.T, p.d, p.k, (int)p.R, s), "combine");
  mark(5, nl, s);
  return st;
}

RouteArgs route_args(const Plan& p, const float* lb, const float* sb, int32_t* idx, float* gates, float* scores) {
  RouteArgs r;
  r.T = p.T;
  r.d = p.d;
  r.E = p.E;
  r.k = p.k;
  r.score = p.score;
  r.renorm = p.renorm;
  r.gate_scale = p.gscale;
  r.logit_bias = lb;
  r.select_bias = p.score == MOE_SCORE_SIGMOID ? sb : nullptr;
  r.idx = idx;
  r.gates = gates;
  r.scores = scores;
  r.tiles_per_block = p.rpb;
  r.n_groups = p.G;
  r.topk_groups = p.GM;
  return r;
}

PermArgs perm_args(const Plan& p, void* ws, int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                   uint8_t* drop) {
  PermArgs a;
  a.T = p.T;
  a.k = p.k;
  a.E = p.E;
  a.cap = (int)p.cap;
  a.counts = counts;
  a.offsets = offsets;
  a.row_token = row_token;
  a.slot_row = slot_row;
  a.drop = drop;
  a.items = at<int4>(ws, p.o_items);
  a.n_items = at<int32_t>(ws, p.o_nitems);
  a.bm = p.bm;
  // the down GEMM's own tile map (many-token path only: the plan splits nowhere else)
  const bool split = p.bm_dn != p.bm;
  a.items_dn = split ? at<int4>(ws, p.o_items_dn) : nullptr;
  a.n_items_dn = split ? at<int32_t>(ws, p.o_nitems_dn) : nullptr;
  a.bm_dn = p.bm_dn;
  a.rt = p.rt * p.rpb;  // tokens per permute block
  return a;
}

moe_status check_experts(const Plan& p, const moe_experts* w) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "experts struct is NULL");
  if (!w->w_gate || !w->w_up || !w->w_down) return fail(MOE_ERR_INVALID_ARG, "routed expert weight pointer is NULL");
  if (!al16(w->w_gate) || !al16(w->w_up) || !al16(w->w_down))
    return fail(MOE_ERR_INVALID_ARG, "routed expert weights must be 16-byte aligned");
  if ((p.wdt == MOE_INT4_G128 || fp8_weights(p.wdt)) && (!w->s_gate || !w->s_up || !w->s_down))
    return fail(MOE_ERR_INVALID_ARG, "INT4 and FP8 experts need s_gate, s_up and s_down");
  if (fp8_weights(p.wdt) && (!al4(w->s_gate) || !al4(w->s_up) || !al4(w->s_down)))
    return fail(MOE_ERR_INVALID_ARG, "FP8 scales must be 4-byte aligned");
  if (p.wdt == MOE_INT4_G128 && (!al2(w->s_gate) || !al2(w->s_up) || !al2(w->s_down)))
    return fail(MOE_ERR_INVALID_ARG, "INT4 scales must be 2-byte aligned");
  if (p.S > 0) {
    if (!w->sh_gate || !w->sh_up || !w->sh_down) return fail(MOE_ERR_INVALID_ARG, "shared expert weight pointer is NULL");
    if (!al16(w->sh_gate) || !al16(w->sh_up) || !al16(w->sh_down))
      return fail(MOE_ERR_INVALID_ARG, "shared expert weights must be 16-byte aligned");
    if (p.wdt == MOE_INT4_G128 && (!w->shs_gate || !w->shs_up || !w->shs_down))
      return fail(MOE_ERR_INVALID_ARG, "INT4 shared experts need shs_gate, shs_up and shs_down");
    if (p.wdt == MOE_INT4_G128 && (!al2(w->shs_gate) || !al2(w->shs_up) || !al2(w->shs_down)))
      return fail(MOE_ERR_INVALID_ARG, "INT4 shared-expert scales must be 2-byte aligned");
    if (fp8_weights(p.wdt) && (!w->shs_gate || !w->shs_up || !w->shs_down))
      return fail(MOE_ERR_INVALID_ARG, "FP8 shared experts need shs_gate, shs_up and shs_down");
    if (fp8_weights(p.wdt) && (!al4(w->shs_gate) || !al4(w->shs_up) || !al4(w->shs_down)))
      return fail(MOE_ERR_INVALID_ARG, "FP8 shared-expert scales must be 4-byte aligned");
  }
  return MOE_OK;
}

FfnArgs ffn_args(const Plan& p, void* ws, const void* x, const int32_t* row_token, const moe_experts* w, void* y,
                 void* ysh) {
  FfnArgs a;
  a.T = p.T;
  a.d = p.d;
  a.E = p.E;
  a.F = p.F;
  a.S = p.S;
  a.FS = p.FS;
  a.R = (int)p.R;
  a.x = x;
  a.row_token = row_token;
  a.items = at<int4>(ws, p.o_items);
  a.n_items = at<int32_t>(ws, p.o_nitems);
  a.items_max = (int)p.items_max;
  a.sh_items = p.sh_items;
  a.bm = p.bm;
  a.wtiled = p.tiled;
  a.wstream = p.wstream;
  a.rowskip_gu = p.rowskip_gu;
  a.rowskip_dn = p.rowskip_dn;
  a.wg = w->w_gate;
  a.wu = w->w_up;
  a.wd = w->w_down;
  a.sg = w->s_gate;
  a.su = w->s_up;
  a.sd = w->s_down;
  a.shg = w->sh_gate;
  a.shu = w->sh_up;
  a.shd = w->sh_down;
  a.shsg = w->shs_gate;
  a.shsu = w->shs_up;
  a.shsd = w->shs_down;
  a.h = at<void>(ws, p.o_h);
  a.hsh = at<void>(ws, p.o_hsh);
  a.y = y;
  a.ysh = ysh;
  return a;
}

// router (logits, scores, top-k, gates) for the planned mode
moe_status enqueue_route(const Plan& p, const void* x, const void* wr, const RouteArgs& ra, void* ws, hipStream_t s) {
  moe_status st;
  if (p.single) {
    float* part = at<float>(ws, p.o_part);
    if ((st = hip_ok(launch_router_partial(p.act, x, wr, p.T, p.d, p.E, p.kchunk, p.KS, part, nullptr, s), "router")))
      return st;
    PermArgs none{};
    return hip_ok(launch_route_small(part, p.KS, ra, nullptr, none, 1, 0, nullptr, s), "route");
  }
  return hip_ok(launch_router_fused(p.act, x, wr, ra, p.rt, at<int32_t>(ws, p.o_hist), s), "router");
}

// ---- the built-in workspace of moe_forward_noalloc
// A file-scope device array, so a forward can run with no allocation at all.  Host code
// never uses the array's name as an address: each device's copy is at its own address,
// looked up once per device with hipGetSymbolAddress and kept in g_scratch.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_validate(const moe_cfg* cfg) {
  Plan p;
  return make_plan(cfg, &p);
}

int64_t moe_rows(const moe_cfg* cfg) {
  Plan p;
  if (make_plan(cfg, &p) != MOE_OK) return -1;
  return p.R;
}

int64_t moe_capacity(const moe_cfg* cfg) {
  Plan p;
  if (make_plan(cfg, &p) != MOE_OK) return -2;
  return p.cap;
}

size_t moe_workspace_bytes(const moe_cfg* cfg) {
  Plan p;
  if (make_plan(cfg, &p) != MOE_OK) return 0;
  return p.total;
}

int32_t moe_forward_launches(const moe_cfg* cfg) {
  Plan p;
  if (make_plan(cfg, &p) != MOE_OK || p.T == 0) return 0;
  return one_token(p) ? 4 : (p.a8 ? 7 : 5);
}

moe_status moe_route(const moe_cfg* cfg, const void* x, const void* w_router, const float* logit_bias,
                     const float* select_bias, int32_t* topk_idx, float* topk_w, float* scores, void* ws,
                     size_t ws_bytes, void* stream) {
  Plan p;
  moe_status st;
  if ((st = make_plan(cfg, &p))) return st;
  if (p.T == 0) return MOE_OK;
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if (!x || !w_router || !topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "NULL x, w_router, topk_idx or topk_w");
  if (!al16(x) || !al16(w_router)) return fail(MOE_ERR_INVALID_ARG, "x and w_router must be 16-byte aligned");
  if (!al4(topk_idx) || !al4(topk_w) || (scores && !al4(scores)) || (logit_bias && !al4(logit_bias)) ||
      (select_bias && !al4(select_bias)))
    return fail(MOE_ERR_INVALID_ARG, "index / fp32 arrays must be 4-byte aligned");
  RouteArgs ra = route_args(p, logit_bias, select_bias, topk_idx, topk_w, scores);
  return enqueue_route(p, x, w_router, ra, ws, (hipStream_t)stream);
}

moe_status moe_permute(const moe_cfg* cfg, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                       int32_t* row_token, int32_t* slot_row, uint8_t* drop_mask, void* ws, size_t ws_bytes,
                       void* stream) {
  Plan p;
  moe_status st;
  if ((st = make_plan(cfg, &p))) return st;
  if (p.T == 0) return MOE_OK;
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if (!topk_idx || !counts || !offsets || !row_token || !slot_row || !drop_mask)
    return fail(MOE_ERR_INVALID_ARG, "NULL permutation argument");
  if (!al4(topk_idx) || !al4(counts) || !al4(offsets) || !al4(row_token) || !al4(slot_row))
    return fail(MOE_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  PermArgs pa = perm_args(p, ws, counts, offsets, row_token, slot_row, drop_mask);
  if (p.single) {
    RouteArgs ra = route_args(p, nullptr, nullptr, nullptr, nullptr, nullptr);
    return hip_ok(launch_route_small(nullptr, 0, ra, topk_idx, pa, 0, 1, nullptr, s), "permute");
  }
  int32_t* hist = at<int32_t>(ws, p.o_hist);
  if ((st = hip_ok(launch_tile_hist(topk_idx, p.T, p.k, p.E, p.rt * p.rpb, hist, s), "histogram"))) return st;
  return hip_ok(launch_permute_multi(topk_idx, hist, pa, s), "permute");
}

moe_status moe_expert_ffn(const moe_cfg* cfg, const void* x, const int32_t* offsets, const int32_t* row_token,
                          const moe_experts* w, void* y_rows, void* y_shared, void* ws, size_t ws_bytes,
                          void* stream) {
  Plan p;
  moe_status st;
  if ((st = make_plan(cfg, &p))) return st;
  if (p.T == 0) return MOE_OK;
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if ((st = check_experts(p, w))) return st;
  if (!x || !offsets || !row_token || !y_rows) return fail(MOE_ERR_INVALID_ARG, "NULL x, offsets, row_token or y_rows");
  if ((p.S > 0) != (y_shared != nullptr)) return fail(MOE_ERR_INVALID_ARG, "y_shared must be given iff n_shared > 0");
  if (!al16(x) || !al16(y_rows) || (y_shared && !al16(y_shared)))
    return fail(MOE_ERR_INVALID_ARG, "x, y_rows and y_shared must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if ((st = hip_ok(launch_tile_map(offsets, p.E, (int)p.R, p.bm, at<int4>(ws, p.o_items), at<int32_t>(ws, p.o_nitems), s),
                   "tile map")))
    return st;
  if (p.bm_dn != p.bm &&
      (st = hip_ok(launch_tile_map(offsets, p.E, (int)p.R, p.bm_dn, at<int4>(ws, p.o_items_dn),
                                   at<int32_t>(ws, p.o_nitems_dn), s),
                   "down tile map")))
    return st;
  FfnArgs a = ffn_args(p, ws, x, row_token, w, y_rows, y_shared);
  if ((st = enqueue_gateup(p, ws, a, s))) return st;
  return enqueue_down(p, ws, down_args(p, ws, a), s);
}

moe_status moe_combine(const moe_cfg* cfg, const void* y_rows, const int32_t* slot_row, const float* topk_w,
                       const void* y_shared, void* out, void* stream) {
  Plan p;
  moe_status st;
  if ((st = make_plan(cfg, &p))) return st;
  if (p.T == 0) return MOE_OK;
  if (!y_rows || !slot_row || !topk_w || !out) return fail(MOE_ERR_INVALID_ARG, "NULL combine argument");
  if ((p.S > 0) != (y_shared != nullptr)) return fail(MOE_ERR_INVALID_ARG, "y_shared must be given iff n_shared > 0");
  if (!al16(y_rows) || !al16(out) || (y_shared && !al16(y_shared)))
    return fail(MOE_ERR_INVALID_ARG, "y_rows, y_shared and out must be 16-byte aligned");
  if (!al4(slot_row) || !al4(topk_w)) return fail(MOE_ERR_INVALID_ARG, "slot_row and topk_w must be 4-byte aligned");
  return hip_ok(launch_combine(p.act, y_rows, slot_row, topk_w, y_shared, out, p.T, p.d, p.k, (int)p.R,
                               (hipStream_t)stream),
                "combine");
}

moe_status moe_forward(const moe_cfg* cfg, const void* x, const void* w_router, const float* logit_bias,
                       const float* select_bias, const moe_experts* w, void* out, int32_t* topk_idx, float* topk_w,
                       uint8_t* drop_mask, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  moe_status st;
  if ((st = make_plan(cfg, &p))) return st;
  if (p.T == 0) return MOE_OK;
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if ((st = check_experts(p, w))) return st;
  if (!x || !w_router || !out || !topk_idx || !topk_w || !drop_mask)
    return fail(MOE_ERR_INVALID_ARG, "NULL x, w_router, out, topk_idx, topk_w or drop_mask");
  if (!al16(x) || !al16(w_router) || !al16(out)) return fail(MOE_ERR_INVALID_ARG, "x, w_router and out must be 16-byte aligned");
  if (!al4(topk_idx) || !al4(topk_w) || (logit_bias && !al4(logit_bias)) || (select_bias && !al4(select_bias)))
    return fail(MOE_ERR_INVALID_ARG, "index / fp32 arrays must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  int32_t* slot = at<int32_t>(ws, p.o_slot);
  int32_t* rowtok = at<int32_t>(ws, p.o_rowtok);
  RouteArgs ra = route_args(p, logit_bias, select_bias, topk_idx, topk_w, nullptr);
  PermArgs pa = perm_args(p, ws, at<int32_t>(ws, p.o_counts), at<int32_t>(ws, p.o_off), rowtok, slot, drop_mask);
  const int nl = one_token(p) ? 4 : 5;
  mark(0, nl, s);
  if (p.single) {
    float* part = at<float>(ws, p.o_part);
    int32_t* arrived = at<int32_t>(ws, p.o_arrived);
    if ((st = hip_ok(launch_router_partial(p.act, x, w_router, p.T, p.d, p.E, p.kchunk, p.KS, part, arrived, s),
                     "router")))
      return st;
    mark(1, nl, s);
    if ((st = hip_ok(launch_route_small(part, p.KS, ra, nullptr, pa, 1, 1, arrived, s), "route/permute"))) return st;
  } else {
    int32_t* hist = at<int32_t>(ws, p.o_hist);
    if ((st = hip_ok(launch_router_fused(p.act, x, w_router, ra, p.rt, hist, s), "router"))) return st;
    mark(1, nl, s);
    if ((st = hip_ok(launch_permute_multi(ra.idx, hist, pa, s), "permute"))) return st;
  }
  mark(2, nl, s);
  void* ysh = p.S ? at<void>(ws, p.o_ysh) : nullptr;
  FfnArgs a = ffn_args(p, ws, x, rowtok, w, at<void>(ws, p.o_y), ysh);
  return enqueue_experts_and_combine(p, ws, a, topk_idx, slot, topk_w, ysh, out, s, true);
}

moe_status moe_forward_noalloc(const moe_cfg* cfg, const void* x, const void* w_router, const float* logit_bias,
                               const float* select_bias, const moe_experts* w, void* out, int32_t* topk_idx,
                               float* topk_w, uint8_t* drop_mask, void* stream) {
  Plan p;
  moe_status st;
  if ((st = make_plan(cfg, &p))) return st;
  if (p.T == 0) return MOE_OK;
  if (p.total > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "this cfg needs %zu workspace bytes; the built-in scratch holds %zu (use moe_forward with a "
                "caller-owned workspace)", p.total, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws))) return st;
  return moe_forward(cfg, x, w_router, logit_bias, select_bias, w, out, topk_idx, topk_w, drop_mask, ws,
                     kScratchBytes, stream);
}

int64_t moe_noalloc_scratch_bytes(void) { return (int64_t)kScratchBytes; }

moe_status moe_forward_with_routes(const moe_cfg* cfg, const void* x, const int32_t* topk_idx, const float* topk_w,
                                   const moe_experts* w, void* out, uint8_t* drop_mask, void* ws, size_t ws_bytes,
                                   void* stream) {
  Plan p;
  moe_status st;
  if ((st = make_plan(cfg, &p))) return st;
  if (p.T == 0) return MOE_OK;
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if ((st = check_experts(p, w))) return st;
  if (!x || !topk_idx || !topk_w || !out || !drop_mask)
    return fail(MOE_ERR_INVALID_ARG, "NULL x, topk_idx, topk_w, out or drop_mask");
  if (!al16(x) || !al16(out)) return fail(MOE_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
  if (!al4(topk_idx) || !al4(topk_w)) return fail(MOE_ERR_INVALID_ARG, "topk_idx and topk_w must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  int32_t* slot = at<int32_t>(ws, p.o_slot);
  int32_t* rowtok = at<int32_t>(ws, p.o_rowtok);
  PermArgs pa = perm_args(p, ws, at<int32_t>(ws, p.o_counts), at<int32_t>(ws, p.o_off), rowtok, slot, drop_mask);
  // the same permutation launches as moe_permute (and so as moe_forward, whose route
  // launch ranks the pairs with the same code)
  if (p.single) {
    RouteArgs ra = route_args(p, nullptr, nullptr, nullptr, nullptr, nullptr);
    if ((st = hip_ok(launch_route_small(nullptr, 0, ra, topk_idx, pa, 0, 1, nullptr, s), "permute"))) return st;
  } else {
    int32_t* hist = at<int32_t>(ws, p.o_hist);
    if ((st = hip_ok(launch_tile_hist(topk_idx, p.T, p.k, p.E, p.rt * p.rpb, hist, s), "histogram"))) return st;
    if ((st = hip_ok(launch_permute_multi(topk_idx, hist, pa, s), "permute"))) return st;
  }
  void* ysh = p.S ? at<void>(ws, p.o_ysh) : nullptr;
  FfnArgs a = ffn_args(p, ws, x, rowtok, w, at<void>(ws, p.o_y), ysh);
  return enqueue_experts_and_combine(p, ws, a, topk_idx, slot, topk_w, ysh, out, s, false);
}

moe_status moe_pack_weights(int32_t dtype, const void* src, void* dst, int64_t rows, int32_t K, void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16 && dtype != MOE_INT4_G128 && !fp8_weights(dtype))
    return fail(MOE_ERR_INVALID_ARG, "dtype=%d is not a moe_dtype", dtype);
  if (rows < 0 || rows % 16) return fail(MOE_ERR_INVALID_ARG, "rows=%lld is not a non-negative multiple of 16", (long long)rows);
  const int64_t rb = dtype == MOE_INT4_G128 ? (int64_t)K / 2
                     : fp8_weights(dtype)     ? (int64_t)K
                                              : (int64_t)K * (dtype == MOE_F32 ? 4 : 2);
  if (K <= 0 || (dtype == MOE_INT4_G128 && K % kInt4Group) || rb % 64)
    return fail(MOE_ERR_INVALID_ARG, "K=%d: a row must be a positive multiple of 64 bytes (INT4: K multiple of 128)", K);
  if (rows == 0) return MOE_OK;
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "NULL src or dst");
  if (!al16(src) || !al16(dst)) return fail(MOE_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  const uintptr_t a0 = (uintptr_t)src, b0 = (uintptr_t)dst, n = (uintptr_t)(rows * rb);
  if (a0 < b0 + n && b0 < a0 + n) return fail(MOE_ERR_INVALID_ARG, "src and dst overlap");
  return hip_ok(launch_pack_tiled(src, dst, rows, rb, (hipStream_t)stream), "pack");
}

moe_status moe_set_timing_events(void* const* events, int32_t n_events) {
  g_events = events;
  g_nevents = events ? n_events : 0;
  return MOE_OK;
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

}  // extern "C"
