// C ABI of the LatentMoE layer forward: argument checks, workspace carving and
// the launch sequence. Host code only; every step of the layer runs in the
// kernels of router.hip, permute.hip, gemm.hip and combine.hip.
#include "../../include/moe_api.h"

#include <string.h>

#include <mutex>

#include "kernels.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Tile shape of the grouped expert products; the permutation lays out the
// M-tile table for this BM.
constexpr int kGroupedCfg = TILE_256x256_GROUPED;
constexpr int kGroupedBM = 256;

// Up to this many tokens the products stream their weights with the skinny
// (few-row) kernels instead of the tiled MFMA GEMM.
constexpr int kSkinnyMaxT = 64;
// Dense skinny products split K until about this many waves are in flight.
#ifndef MOE_SKINNY_TARGET_WAVES
#define MOE_SKINNY_TARGET_WAVES 2048
#endif
#ifndef MOE_SKINNY_KSPLIT_DIV
#define MOE_SKINNY_KSPLIT_DIV 4
#endif
constexpr int kSkinnyTargetWaves = MOE_SKINNY_TARGET_WAVES;
// tokens from which the tiled router product splits K in two
constexpr int kRouterSplitMinT = 4096;

// bf16 products of 1-16 rows aim at twice as many waves: one token's products
// gained about 1 % from it, while the fp32 router product lost (its waves
// carry three times the bytes per column).
int skinny_ksplit(int N, int K, int M, bool f32_weights = false) {
  if (N <= 0 || K < 64) return 1;
  const int width = M > 16 ? 64 : 16;      // columns per wave (see skinny_slabs_per_wave)
  const int slabs = (N + width - 1) / width;
  const int target = (M <= 16 && !f32_weights) ? 2 * kSkinnyTargetWaves : kSkinnyTargetWaves;
  int ks = (target + slabs - 1) / slabs;
  // the fp32 partials are written once and read once: 8*ks*M*N bytes against
  // 2*N*K bytes of weights; keep them within the weight traffic (a quarter of
  // it left a 64-token decode's dense products with 64-256 waves: measured
  // 12-42 % slower per product)
  const int cap = std::max(1, K / (MOE_SKINNY_KSPLIT_DIV * std::max(M, 1)));
  ks = std::max(1, std::min(std::min(ks, cap), K / 64));   // whole 64-deep steps per split
  return ks;
}

struct Layout {
  // route
  size_t wsplit, logits;
  // permute
  size_t masks, base, counts, tile_info, n_mtiles, touched, n_touched, gemm_ctr;
  // forward
  size_t idx, gate, gap, offsets, row_token, slot_row, z, hs, h, y, y_lat, partial;
  size_t route_end, permute_begin, permute_end, total;
  int64_t ldl;         // logits row stride (E rounded up to 64)
  int nblk;            // token blocks of 64
  int max_mtiles;      // M-tile table capacity
};

// Which fields of moe_dims a call reads.
enum DimsUse { USE_ROUTE = 1, USE_PERMUTE = 2, USE_ALL = 3 };

// Group-limited routing: 0 in either field means the plain top-K (1 group).
int groups_of(const moe_dims& d) { return d.n_group == 0 ? 1 : d.n_group; }
int topk_groups_of(const moe_dims& d) { return d.topk_group == 0 ? 1 : d.topk_group; }

bool dims_ok(const moe_dims* d, int* status, int use = USE_ALL) {
  *status = MOE_ERR_INVALID;
  if (d == nullptr) return false;
  if (d->T <= 0 || d->E <= 0 || d->K <= 0 || d->K > d->E) return false;
  if ((use & USE_ROUTE) && d->H <= 0) return false;
  if (use == USE_ALL && (d->L <= 0 || d->I <= 0 || d->Is <= 0)) return false;
  if (use & USE_ROUTE) {
    const int ng = groups_of(*d), tg = topk_groups_of(*d);
    if (ng < 1 || tg < 1 || tg > ng || d->E % ng) return false;
    if ((int64_t)d->K > (int64_t)tg * (d->E / ng)) return false;
  }
  *status = MOE_ERR_UNSUPPORTED;
  if ((use & USE_ROUTE) && groups_of(*d) > kMaxGroups) return false;
  if (d->E > kMaxExperts || d->K > kMaxTopK) return false;
  if ((use & USE_ROUTE) && d->H % 64) return false;
  if (use == USE_ALL && (d->L % 64 || d->I % 64 || d->Is % 64)) return false;
  // permuted rows are indexed with int32; byte offsets of one tensor stay below 2^40
  const int64_t tk = (int64_t)d->T * d->K;
  if (tk > (int64_t)0x7FFFFFFF) return false;
  // the expert up product gathers rows of z [T, L] through 32-bit byte offsets
  if (use == USE_ALL && (int64_t)d->T * d->L * 2 >= ((int64_t)1 << 32)) return false;
  *status = MOE_OK;
  return true;
}

// moe_dims with the fields a partial call does not read zeroed, for the layout.
moe_dims only_used(const moe_dims& d, int use) {
  moe_dims u = d;
  if (!(use & USE_ROUTE)) { u.H = 0; u.n_group = 0; u.topk_group = 0; }
  if (use != USE_ALL) { u.L = 0; u.I = 0; u.Is = 0; }
  return u;
}

// The tiled router product from kRouterSplitMinT tokens splits K in two. With
// at most 128 experts (E a multiple of 64) it also takes the three bf16 parts
// of the weight as 3E output columns instead of three K segments of one
// accumulator (the parts are stored one after the other, so their rows are one
// [3E, H] matrix): three times the workgroups, each a third of the k steps.
// The top-k adds the 2 x 3 partial logits. (E = 128 gives only T/128 x 2
// workgroups otherwise: 7-14 % MFMA busy at 4096-8192 tokens.)
bool router_splits_k(int64_t T, int64_t H) { return T >= kRouterSplitMinT && H % 128 == 0; }
bool router_stacks_parts(int64_t T, int64_t H, int64_t E) {
  return router_splits_k(T, H) && E <= 128 && E % 64 == 0;
}

Layout make_layout(const moe_dims& d) {
  Layout l{};
  const int64_t T = d.T, H = d.H, L = d.L, E = d.E, I = d.I, K = d.K, Is = d.Is, TK = T * K;
  l.ldl = (E + 63) / 64 * 64;
  l.nblk = (int)((T + 63) / 64);
  l.max_mtiles = (int)(TK / kGroupedBM + E + 1);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  // a forward of at most kSkinnyMaxT tokens splits the router weight in
  // registers (no parts); moe_route (L = I = Is = 0 here) always tiles
  const bool few = T <= kSkinnyMaxT && L > 0 && I > 0 && Is > 0 && H > 0;
  l.wsplit = take(few ? 0 : 3 * E * H * 2);
  // two halves when the router product splits K, each 3 column blocks when it stacks the weight parts
  l.logits = take(2 * T * l.ldl * 4 * (router_stacks_parts(T, H, E) ? 3 : 1));
  l.route_end = o;
  l.permute_begin = o;
  l.masks = take(E * l.nblk * 8);
  l.base = take(E * l.nblk * 4);
  l.counts = take(E * 4);
  l.tile_info = take((size_t)l.max_mtiles * 16);
  l.n_mtiles = take(4);
  l.touched = take(E * 4);
  l.n_touched = take(4);
  l.gemm_ctr = take(kGemmCounters * 4);
  l.permute_end = o;
  l.idx = take(TK * 4);
  l.gate = take(TK * 4);
  l.gap = take(T * 4);
  l.offsets = take((E + 1) * 4);
  l.row_token = take(TK * 4);
  l.slot_row = take(TK * 4);
  l.z = take(T * L * 2);
  l.hs = take(T * Is * 2);
  l.h = take(TK * I * 2);
  l.y = take(TK * L * 2);
  l.y_lat = take(T * L * 2);
  l.partial = o;
  if (few) {
    // split-K partials of the dense skinny products: [ksplit, T, N] fp32
    size_t p = 0;
    p = std::max(p, (size_t)skinny_ksplit((int)l.ldl, (int)(3 * H), (int)T, true) * T * l.ldl * 4);
    p = std::max(p, (size_t)skinny_ksplit((int)L, (int)H, (int)T) * T * L * 4);
    p = std::max(p, (size_t)skinny_ksplit((int)Is, (int)H, (int)T) * T * Is * 4);
    p = std::max(p, (size_t)skinny_ksplit((int)H, (int)(L + Is), (int)T) * T * H * 4);
    take(p);
  }
  l.total = o;
  return l;
}

template <typename P>
P* at(void* ws, size_t off) { return reinterpret_cast<P*>(static_cast<char*>(ws) + off); }

bool ws_ok(const void* ws, size_t have, size_t need) {
  return ws != nullptr && have >= need && (reinterpret_cast<uintptr_t>(ws) % kAlign) == 0;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Dense problem: C[M, N] = epi(sum_s A_s . B_s^T).
GemmProblem dense_problem(int cfg, int M, int N, int Nb, void* C, int64_t ldc, int epi) {
  GemmProblem p{};
  const TileShape ts = tile_shape(cfg);
  p.a_records = kRsrc2G;
  p.M = M;
  p.N = N;
  p.Nb = Nb;
  p.C = C;
  p.ldc = ldc;
  p.epi = epi;
  p.mtiles = (M + ts.BM - 1) / ts.BM;
  p.ntiles = (N + ts.BN - 1) / ts.BN;
  p.group_m = 4;
  return p;
}

void add_seg(GemmProblem& p, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int K) {
  p.seg[p.nseg++] = KSeg{A, B, lda, ldb, K};
}

void add_seg(SkinnyProblem& p, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int K) {
  p.seg[p.nseg++] = KSeg{A, B, lda, ldb, K};
}

// Dense skinny problem C[M, N] over a total reduction length Ktot.
SkinnyProblem skinny_dense(int M, int N, int Nb, void* C, int64_t ldc, int epi, int Ktot, float* partial,
                           bool f32_weights = false) {
  SkinnyProblem p{};
  p.M = M;
  p.N = N;
  p.Nb = Nb;
  p.groups = 1;
  p.C = C;
  p.ldc = ldc;
  p.epi = epi;
  p.ksplit = skinny_ksplit(N, Ktot, M, f32_weights);
  p.partial = p.ksplit > 1 ? partial : nullptr;
  if (p.partial == nullptr) p.ksplit = 1;
  return p;
}

// Grouped skinny problem over the permuted rows of each expert that has tokens;
// at most min(E, T*K) experts can.
SkinnyProblem skinny_grouped(int max_groups, const PermuteScratch& ps, int N, const int32_t* offsets,
                             const int32_t* gather, int64_t b_estride, void* C, int64_t ldc, int epi) {
  SkinnyProblem p{};
  p.N = N;
  p.Nb = N;
  p.groups = max_groups;
  p.group_list = ps.touched;
  p.n_groups = ps.n_touched;
  p.offsets = offsets;
  p.gather = gather;
  p.b_estride = b_estride;
  p.C = C;
  p.ldc = ldc;
  p.epi = epi;
  p.ksplit = 1;
  return p;
}

// 256x256 tiles when the launch's tiles of that size (col_tiles 256-column
// tiles over all its problems) fill the 256 CUs in whole waves, the last at
// least 80 % full; else smaller tiles (the router's N = E is narrow, decode's M
// is a few rows). Dense products alone, 256x256 against 128x128: 1.32 against
// 1.08 PFLOP/s at 256 tiles (one wave), 1.18 / 1.07 at 640, 1.33 / 1.05 at
// 1536; 1.00 / 1.07 at 320 and 0.94 / 1.08 at 128.
int choose_dense_cfg(int M, int N, int col_tiles) {
  const int64_t t = (int64_t)((M + 255) / 256) * col_tiles;
  if (M >= 256 && N >= 256 && t >= 256 && t * 5 >= (t + 255) / 256 * 256 * 4) return TILE_256x256;
  if (M <= 64 && N >= 256) return TILE_64x256;
  return TILE_128x128;
}
int col_tiles256(int N) { return (N + 255) / 256; }

// Records events[phase] (if any) on the stream.
struct Marks {
  hipEvent_t* ev;
  hipStream_t st;
  hipError_t mark(int phase) const { return ev ? hipEventRecord(ev[phase], st) : hipSuccess; }
};

int run_route(const moe_dims& d, const Layout& l, const uint16_t* x, const float* w_router, const float* bias,
              int32_t* idx, float* gate, float* gap, void* ws, hipStream_t st, const Marks& mk = Marks{nullptr, 0},
              float* partial = nullptr) {
  uint16_t* parts = at<uint16_t>(ws, l.wsplit);
  float* logits = at<float>(ws, l.logits);
  const float* logits2 = nullptr;
  int64_t ldl = l.ldl;                       // row length of the logits the top-k reads
  int nparts = 1;                            // column blocks of E summed per half (stacked parts)
  const bool skinny = d.T <= kSkinnyMaxT && partial != nullptr;
  hipError_t e = hipSuccess;
  if (mk.mark(MOE_PHASE_ROUTER_SPLIT) != hipSuccess) return MOE_ERR_HIP;
  // the tiled GEMM reads the fp32 weight as three bf16 parts written here; the
  // few-token product splits it in registers instead (no pass, 16 instead of
  // 24 + 16 bytes of traffic per weight)
  if (!skinny) e = launch_split_router_weight(w_router, d.E, d.H, parts, st);
  if (e != hipSuccess) return MOE_ERR_HIP;
  const int64_t EH = (int64_t)d.E * d.H;
  if (mk.mark(MOE_PHASE_ROUTER_GEMM) != hipSuccess) return MOE_ERR_HIP;
  int fused_ksplit = 0;                      // > 0: the top-K sums the product's partials itself
  if (skinny) {
    SkinnyProblem P = skinny_dense(d.T, (int)l.ldl, d.E, logits, l.ldl, EPI_F32, d.H, partial, true);
    add_seg(P, x, d.H, nullptr, d.H, d.H);
    P.f32_b = w_router;
    if (P.partial != nullptr) fused_ksplit = P.ksplit;
    e = launch_skinny(P, st, fused_ksplit == 0);
  } else if (router_splits_k(d.T, d.H)) {
    // Many tokens: K split in two (each half of H over the three weight parts)
    // so that more tiles fill the CUs (E = 512 columns make only 2 column
    // tiles of 256); the top-k adds the halves' fp32 logits. Ultra prefill:
    // 0.43 ms with 128x128 tiles over the whole K. Up to 128 experts take
    // 128x128 tiles: a 256-wide tile would issue twice the work on padding
    // columns with half as many workgroups (counters: 7-15 % MFMA busy at
    // 4096-8192 tokens, E = 128).
    const int Hh = d.H / 2;
    const int cfg = l.ldl <= 128 ? TILE_128x128 : TILE_256x256;
    const bool stack = router_stacks_parts(d.T, d.H, d.E);
    if (stack) {
      ldl = 3 * (int64_t)d.E;
      nparts = 3;
    }
    GemmLaunch L{};
    L.np = 2;
    for (int h = 0; h < 2; ++h) {
      L.p[h] = dense_problem(cfg, d.T, (int)ldl, stack ? (int)ldl : d.E, logits + (int64_t)h * d.T * ldl, ldl, EPI_F32);
      if (stack) add_seg(L.p[h], x + h * Hh, d.H, parts + h * Hh, d.H, Hh);
      else
        for (int s = 0; s < 3; ++s) add_seg(L.p[h], x + h * Hh, d.H, parts + s * EH + h * Hh, d.H, Hh);
    }
    e = launch_gemm(L, cfg, st);
    logits2 = logits + (int64_t)d.T * ldl;
  } else {
    const int cfg = choose_dense_cfg(d.T, (int)l.ldl, col_tiles256((int)l.ldl));
    GemmLaunch L{};
    L.np = 1;
    L.p[0] = dense_problem(cfg, d.T, (int)l.ldl, d.E, logits, l.ldl, EPI_F32);
    for (int s = 0; s < 3; ++s) add_seg(L.p[0], x, d.H, parts + s * EH, d.H, d.H);
    e = launch_gemm(L, cfg, st);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (mk.mark(MOE_PHASE_TOPK) != hipSuccess) return MOE_ERR_HIP;
  if (fused_ksplit > 0)
    e = launch_topk_partials(partial, fused_ksplit, d.T, l.ldl, bias, d.E, d.K, d.routed_scaling, groups_of(d),
                             topk_groups_of(d), idx, gate, gap, st);
  else  // (stacked weight parts lie E columns apart in a logit row)
    e = launch_topk(logits, logits2, ldl, nparts, d.E, bias, d.T, d.E, d.K, d.routed_scaling, groups_of(d),
                    topk_groups_of(d), idx, gate, gap, st);
  return hip_status(e);
}

// The permute scratch of a workspace whose first byte sits at layout offset `origin`.
PermuteScratch permute_scratch(const Layout& l, void* ws, size_t origin) {
  return PermuteScratch{at<uint64_t>(ws, l.masks - origin), at<int32_t>(ws, l.base - origin),
                        at<int32_t>(ws, l.counts - origin),   at<int32_t>(ws, l.tile_info - origin),
                        at<int32_t>(ws, l.n_mtiles - origin),
                        at<int32_t>(ws, l.touched - origin),  at<int32_t>(ws, l.n_touched - origin),
                        at<int32_t>(ws, l.gemm_ctr - origin)};
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return 105; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID:
      return "invalid argument (null pointer, non-positive size, K > E, bad row length or bad expert groups)";
    case MOE_ERR_UNSUPPORTED:
      return "unsupported size (H, L, I, Is must be multiples of 64; E <= 1024; K <= 64; T*K < 2^31; "
             "2*T*L < 2^32; n_group <= 64)";
    case MOE_ERR_WORKSPACE: return "workspace null, too small or not 256-byte aligned";
    case MOE_ERR_HIP: return "HIP launch error";
    case MOE_ERR_TOO_LARGE:
      return "the forward needs more workspace than the allocation-free entry point's static scratch (128 MiB)";
    default: return "unknown status";
  }
}

size_t moe_route_workspace_bytes(const moe_dims* dims) {
  int st;
  if (!dims_ok(dims, &st, USE_ROUTE)) return 0;
  return make_layout(only_used(*dims, USE_ROUTE)).route_end;
}

size_t moe_permute_workspace_bytes(const moe_dims* dims) {
  int st;
  if (!dims_ok(dims, &st, USE_PERMUTE)) return 0;
  const Layout l = make_layout(only_used(*dims, USE_PERMUTE));
  return l.permute_end - l.permute_begin;
}

size_t moe_workspace_bytes(const moe_dims* dims) {
  int st;
  if (!dims_ok(dims, &st)) return 0;
  return make_layout(*dims).total;
}

int moe_workspace_layout(const moe_dims* dims, moe_ws_layout* out) {
  int st;
  if (!dims_ok(dims, &st)) return st;
  if (out == nullptr) return MOE_ERR_INVALID;
  const Layout l = make_layout(*dims);
  out->idx = l.idx;
  out->gate = l.gate;
  out->gap = l.gap;
  out->offsets = l.offsets;
  out->row_token = l.row_token;
  out->slot_row = l.slot_row;
  out->z = l.z;
  out->h = l.h;
  out->y = l.y;
  out->y_lat = l.y_lat;
  out->hs = l.hs;
  out->total = l.total;
  return MOE_OK;
}

int moe_route(const moe_dims* dims, const uint16_t* x, const float* w_router, const float* corr_bias,
              int32_t* topk_idx, float* topk_gate, float* topk_gap, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  int st;
  if (!dims_ok(dims, &st, USE_ROUTE)) return st;
  if (!x || !w_router || !corr_bias || !topk_idx || !topk_gate) return MOE_ERR_INVALID;
  const Layout l = make_layout(only_used(*dims, USE_ROUTE));
  if (!ws_ok(ws, ws_bytes, l.route_end)) return MOE_ERR_WORKSPACE;
  return run_route(*dims, l, x, w_router, corr_bias, topk_idx, topk_gate, topk_gap, ws, stream);
}

int moe_permute(const moe_dims* dims, const int32_t* topk_idx, const uint16_t* src, int32_t C, uint16_t* dst,
                int32_t* expert_offsets, int32_t* row_token, int32_t* slot_row, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  int st;
  if (!dims_ok(dims, &st, USE_PERMUTE)) return st;
  if (!topk_idx || !expert_offsets || !row_token || !slot_row) return MOE_ERR_INVALID;
  if ((src == nullptr) != (dst == nullptr)) return MOE_ERR_INVALID;
  if (src != nullptr && (C <= 0 || C % 8 != 0)) return MOE_ERR_INVALID;
  const Layout l = make_layout(only_used(*dims, USE_PERMUTE));
  const size_t need = l.permute_end - l.permute_begin;
  if (!ws_ok(ws, ws_bytes, need)) return MOE_ERR_WORKSPACE;
  // the caller's workspace holds only the permute scratch
  hipError_t e = launch_permute_maps(topk_idx, dims->T, dims->K, dims->E, kGroupedBM,
                                     permute_scratch(l, ws, l.permute_begin),
                                     expert_offsets, row_token, slot_row, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (src != nullptr)
    e = launch_gather_rows(src, C, row_token, expert_offsets + dims->E, (int64_t)dims->T * dims->K, dst, stream);
  return hip_status(e);
}

}  // extern "C"

namespace {

// mx: MX (MXFP8 or MXFP4) expert weights (then w->w_up / w->w_down are not read), or null.
// The block around the layer: x_in is normed into the workspace (after the
// layer's own scratch) and is the residual of the output.
struct BlockArgs {
  const uint16_t* x_in;
  const uint16_t* gamma;
  float eps;
};

size_t block_extra_bytes(const moe_dims& d) { return align_up((size_t)d.T * d.H * 2); }

bool eps_ok(float eps) { return eps >= 0.f && eps <= 1e30f; }   // also rejects NaN

int forward_impl(const moe_dims* dims, const moe_weights* w, const uint16_t* x, uint16_t* out, void* ws,
                 size_t ws_bytes, hipStream_t stream, const Marks& mk, const moe_experts_mx* mx = nullptr,
                 const BlockArgs* blk = nullptr) {
  int st;
  if (!dims_ok(dims, &st)) return st;
  if (blk != nullptr) {
    if (!blk->x_in || !blk->gamma || !eps_ok(blk->eps)) return MOE_ERR_INVALID;
    if (((uintptr_t)blk->x_in | (uintptr_t)blk->gamma) & 15) return MOE_ERR_INVALID;
    x = blk->x_in;                                  // checked below; replaced by the normed rows
  }
  if (!w || !x || !out || !w->w_router || !w->corr_bias || !w->w_fc1 || !w->w_fc2 || !w->w_sh_up || !w->w_sh_down)
    return MOE_ERR_INVALID;
  {
    // 16-byte loads and stores per lane
    uintptr_t a = (uintptr_t)x | (uintptr_t)out | (uintptr_t)w->w_router | (uintptr_t)w->w_fc1 |
                  (uintptr_t)w->w_fc2 | (uintptr_t)w->w_sh_up | (uintptr_t)w->w_sh_down;
    if (mx == nullptr) a |= (uintptr_t)w->w_up | (uintptr_t)w->w_down;
    if (a & 15) return MOE_ERR_INVALID;
  }
  if (mx != nullptr) {
    if (!mx->w_up || !mx->w_up_scale || !mx->w_down || !mx->w_down_scale) return MOE_ERR_INVALID;
    if (mx->format != 0 && mx->format != 1) return MOE_ERR_INVALID;
    if (((uintptr_t)mx->w_up | (uintptr_t)mx->w_down) & 15) return MOE_ERR_INVALID;
    if (dims->T > kSkinnyMaxT) return MOE_ERR_UNSUPPORTED;   // the tiled expert products take bf16 only
  } else if (!w->w_up || !w->w_down) {
    return MOE_ERR_INVALID;
  }
  const moe_dims& d = *dims;
  const Layout l = make_layout(d);
  if (!ws_ok(ws, ws_bytes, l.total + (blk ? block_extra_bytes(d) : 0))) return MOE_ERR_WORKSPACE;
  const uint16_t* residual = nullptr;
  if (blk != nullptr) {
    // 0. the pre-norm: x = RMSNorm(x_in) into the workspace; x_in is the residual
    uint16_t* xn = at<uint16_t>(ws, l.total);
    if (launch_rmsnorm(blk->x_in, blk->gamma, d.T, d.H, blk->eps, xn, stream) != hipSuccess) return MOE_ERR_HIP;
    x = xn;
    residual = blk->x_in;
  }
  const int64_t T = d.T, H = d.H, L = d.L, I = d.I, Is = d.Is, TK = T * d.K;

  int32_t* idx = at<int32_t>(ws, l.idx);
  float* gate = at<float>(ws, l.gate);
  int32_t* offsets = at<int32_t>(ws, l.offsets);
  int32_t* row_token = at<int32_t>(ws, l.row_token);
  int32_t* slot_row = at<int32_t>(ws, l.slot_row);
  uint16_t* z = at<uint16_t>(ws, l.z);
  uint16_t* hs = at<uint16_t>(ws, l.hs);
  uint16_t* h = at<uint16_t>(ws, l.h);
  uint16_t* y = at<uint16_t>(ws, l.y);
  uint16_t* y_lat = at<uint16_t>(ws, l.y_lat);

  // 1. router
  const bool skinny = d.T <= kSkinnyMaxT;
  float* partial = skinny ? at<float>(ws, l.partial) : nullptr;
  int rc = run_route(d, l, x, w->w_router, w->corr_bias, idx, gate, at<float>(ws, l.gap), ws, stream, mk, partial);
  if (rc != MOE_OK) return rc;

  // 2. permutation maps and the M-tile table of the grouped products
  const PermuteScratch ps = permute_scratch(l, ws, 0);
  if (mk.mark(MOE_PHASE_PERMUTE) != hipSuccess) return MOE_ERR_HIP;
  if (launch_permute_maps(idx, d.T, d.K, d.E, kGroupedBM, ps, offsets, row_token, slot_row, stream) != hipSuccess)
    return MOE_ERR_HIP;

  // 3. x read by one launch for fc1 (z) and the shared expert's up + relu^2 (hs)
  if (skinny) {
    if (mk.mark(MOE_PHASE_FC1_SHARED_UP) != hipSuccess) return MOE_ERR_HIP;
    SkinnyProblem P = skinny_dense(d.T, d.L, d.L, z, L, EPI_BF16, d.H, partial);
    add_seg(P, x, H, w->w_fc1, H, d.H);
    SkinnyProblem Q = skinny_dense(d.T, d.Is, d.Is, hs, Is, EPI_RELU2_BF16, d.H, partial);
    add_seg(Q, x, H, w->w_sh_up, H, d.H);
    if (d.T <= kWgkMaxRows) {
      // both products in one launch, K split inside each workgroup
      if (launch_skinny_wgk(P, &Q, stream) != hipSuccess) return MOE_ERR_HIP;
    } else {
      if (launch_skinny(P, stream) != hipSuccess) return MOE_ERR_HIP;
      if (launch_skinny(Q, stream) != hipSuccess) return MOE_ERR_HIP;
    }
  } else {
    const int cfg = choose_dense_cfg(d.T, std::min(d.L, d.Is), col_tiles256(d.L) + col_tiles256(d.Is));
    GemmLaunch G{};
    G.np = 2;
    G.p[0] = dense_problem(cfg, d.T, d.L, d.L, z, L, EPI_BF16);
    add_seg(G.p[0], x, H, w->w_fc1, H, d.H);
    G.p[1] = dense_problem(cfg, d.T, d.Is, d.Is, hs, Is, EPI_RELU2_BF16);
    add_seg(G.p[1], x, H, w->w_sh_up, H, d.H);
    // rasters of 2 M tiles: Ultra prefill 2.68 -> 2.63 ms (4 is best for the
    // other dense products: fc2 + shared down 2.54 ms against 2.61 with 2)
    G.p[0].group_m = G.p[1].group_m = 2;
    if (mk.mark(MOE_PHASE_FC1_SHARED_UP) != hipSuccess) return MOE_ERR_HIP;
    if (launch_gemm(G, cfg, stream) != hipSuccess) return MOE_ERR_HIP;
  }

  // 4. expert up + relu^2 over the permuted rows; z rows gathered on load
  if (skinny) {
    if (mk.mark(MOE_PHASE_EXPERT_UP) != hipSuccess) return MOE_ERR_HIP;
    SkinnyProblem P = skinny_grouped(std::min(d.E, d.T * d.K), ps, d.I, offsets, row_token, I * L, h, I,
                                     EPI_RELU2_BF16);
    add_seg(P, z, L, mx ? nullptr : w->w_up, L, d.L);
    if (mx) { P.mx_codes = mx->w_up; P.mx_scales = mx->w_up_scale; P.mx_fp4 = mx->format == 1; }
    if (launch_skinny(P, stream) != hipSuccess) return MOE_ERR_HIP;
  } else {
    const TileShape ts = tile_shape(kGroupedCfg);
    GemmLaunch G{};
    G.np = 1;
    GemmProblem& p = G.p[0];
    p.N = d.I;
    p.Nb = d.I;
    p.gather = row_token;
    // gathered z rows are addressed from z's base: past 2 GiB the full 32-bit range
    p.a_records = T * L * 2 > (int64_t)kRsrc2G ? kRsrc4G : kRsrc2G;
    p.tile_info = ps.tile_info;
    p.n_mtiles = ps.n_mtiles;
    p.offsets = offsets;
    p.b_estride = I * L;
    p.C = h;
    p.ldc = I;
    p.epi = EPI_RELU2_BF16;
    p.mtiles = l.max_mtiles;
    p.ntiles = (d.I + ts.BN - 1) / ts.BN;
    // an expert's M tiles side by side for each weight panel (all of them):
    // the gathered latent rows they re-read stay in the Infinity Cache
    p.group_m = 1 << 20;
    add_seg(p, z, L, w->w_up, L, d.L);
    G.counters = ps.gemm_ctr;                  // the XCD tails' counters, zeroed by the permutation
    if (mk.mark(MOE_PHASE_EXPERT_UP) != hipSuccess) return MOE_ERR_HIP;
    if (launch_gemm(G, kGroupedCfg, stream) != hipSuccess) return MOE_ERR_HIP;
  }

  // 5. expert down over the permuted rows
  if (skinny) {
    if (mk.mark(MOE_PHASE_EXPERT_DOWN) != hipSuccess) return MOE_ERR_HIP;
    SkinnyProblem P = skinny_grouped(std::min(d.E, d.T * d.K), ps, d.L, offsets, nullptr, L * I, y, L, EPI_BF16);
    add_seg(P, h, I, mx ? nullptr : w->w_down, I, d.I);
    if (mx) { P.mx_codes = mx->w_down; P.mx_scales = mx->w_down_scale; P.mx_fp4 = mx->format == 1; }
    if (launch_skinny(P, stream) != hipSuccess) return MOE_ERR_HIP;
  } else {
    const TileShape ts = tile_shape(kGroupedCfg);
    GemmLaunch G{};
    G.np = 1;
    GemmProblem& p = G.p[0];
    p.N = d.L;
    p.Nb = d.L;
    p.a_records = kRsrc2G;
    p.tile_info = ps.tile_info;
    p.n_mtiles = ps.n_mtiles;
    p.offsets = offsets;
    p.b_estride = L * I;
    p.C = y;
    p.ldc = L;
    p.epi = EPI_BF16;
    p.mtiles = l.max_mtiles;
    p.ntiles = (d.L + ts.BN - 1) / ts.BN;
    // rasters of 8 M tiles inside an expert: a panel of h rows is read by the
    // expert's 8 column tiles together, not once per column tile when the
    // expert has many M tiles (h, 0.7-3.7 GB, is too large for the Infinity
    // Cache; Super's hottest expert has 31 M tiles: 1.48 -> 1.35 ms; 2, 4 and 8
    // alike, Ultra prefill and Nano unchanged)
    p.group_m = 8;
    add_seg(p, h, I, w->w_down, I, d.I);
    G.counters = ps.gemm_ctr + 8;              // the XCD tails' counters, zeroed by the permutation
    if (mk.mark(MOE_PHASE_EXPERT_DOWN) != hipSuccess) return MOE_ERR_HIP;
    if (launch_gemm(G, kGroupedCfg, stream) != hipSuccess) return MOE_ERR_HIP;
  }

  // 6. gate-weighted combine in the latent
  if (mk.mark(MOE_PHASE_COMBINE) != hipSuccess) return MOE_ERR_HIP;
  if (launch_combine(y, gate, slot_row, d.T, d.K, d.L, y_lat, stream) != hipSuccess) return MOE_ERR_HIP;

  // 7. out = y_lat . W_fc2^T + hs . W_sd^T, one fp32 accumulator, one rounding
  if (skinny) {
    if (mk.mark(MOE_PHASE_FC2_SHARED_DOWN) != hipSuccess) return MOE_ERR_HIP;
    SkinnyProblem P = skinny_dense(d.T, d.H, d.H, out, H, EPI_BF16, d.L + d.Is, partial);
    P.residual = residual;
    P.ldr = H;
    add_seg(P, y_lat, L, w->w_fc2, L, d.L);
    add_seg(P, hs, Is, w->w_sh_down, Is, d.Is);
    if ((d.T <= kWgkMaxRows ? launch_skinny_wgk(P, nullptr, stream) : launch_skinny(P, stream)) != hipSuccess)
      return MOE_ERR_HIP;
  } else {
    const int cfg = choose_dense_cfg(d.T, d.H, col_tiles256(d.H));
    GemmLaunch G{};
    G.np = 1;
    G.p[0] = dense_problem(cfg, d.T, d.H, d.H, out, H, EPI_BF16);
    G.p[0].residual = residual;
    G.p[0].ldr = H;
    add_seg(G.p[0], y_lat, L, w->w_fc2, L, d.L);
    add_seg(G.p[0], hs, Is, w->w_sh_down, Is, d.Is);
    if (mk.mark(MOE_PHASE_FC2_SHARED_DOWN) != hipSuccess) return MOE_ERR_HIP;
    if (launch_gemm(G, cfg, stream) != hipSuccess) return MOE_ERR_HIP;
  }
  if (mk.mark(MOE_N_PHASES) != hipSuccess) return MOE_ERR_HIP;
  (void)TK;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* x, uint16_t* out, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  return forward_impl(dims, w, x, out, ws, ws_bytes, stream, Marks{nullptr, stream});
}

int moe_forward_profiled(const moe_dims* dims, const moe_weights* w, const uint16_t* x, uint16_t* out, void* ws,
                         size_t ws_bytes, hipStream_t stream, hipEvent_t* events, int n_events) {
  if (events == nullptr || n_events < MOE_N_PHASES + 1) return MOE_ERR_INVALID;
  for (int i = 0; i <= MOE_N_PHASES; ++i)
    if (events[i] == nullptr) return MOE_ERR_INVALID;
  return forward_impl(dims, w, x, out, ws, ws_bytes, stream, Marks{events, stream});
}

int moe_forward_mx(const moe_dims* dims, const moe_weights* w, const moe_experts_mx* mx, const uint16_t* x,
                   uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (mx == nullptr) return MOE_ERR_INVALID;
  return forward_impl(dims, w, x, out, ws, ws_bytes, stream, Marks{nullptr, stream}, mx);
}

int moe_forward_mx_profiled(const moe_dims* dims, const moe_weights* w, const moe_experts_mx* mx, const uint16_t* x,
                            uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* events,
                            int n_events) {
  if (mx == nullptr || events == nullptr || n_events < MOE_N_PHASES + 1) return MOE_ERR_INVALID;
  for (int i = 0; i < MOE_N_PHASES + 1; ++i)
    if (events[i] == nullptr) return MOE_ERR_INVALID;
  return forward_impl(dims, w, x, out, ws, ws_bytes, stream, Marks{events, stream}, mx);
}

int moe_quantize_mxfp4(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                       hipStream_t stream) {
  if (rows <= 0 || cols <= 0 || cols % 32) return MOE_ERR_INVALID;
  if (src == nullptr || codes == nullptr || scales == nullptr) return MOE_ERR_INVALID;
  if (((uintptr_t)src | (uintptr_t)codes) & 15) return MOE_ERR_INVALID;
  return hip_status(launch_mxfp4_quantize(src, rows * (cols / 32), codes, scales, stream));
}

int moe_rmsnorm(const uint16_t* x, const uint16_t* gamma, int64_t T, int32_t H, float eps, uint16_t* y,
                hipStream_t stream) {
  if (x == nullptr || gamma == nullptr || y == nullptr || T <= 0 || H <= 0 || H % 8 || !eps_ok(eps))
    return MOE_ERR_INVALID;
  if (((uintptr_t)x | (uintptr_t)gamma | (uintptr_t)y) & 15) return MOE_ERR_INVALID;
  return hip_status(launch_rmsnorm(x, gamma, T, H, eps, y, stream));
}

size_t moe_block_workspace_bytes(const moe_dims* dims) {
  int st;
  if (!dims_ok(dims, &st)) return 0;
  return make_layout(*dims).total + block_extra_bytes(*dims);
}

int moe_block_forward(const moe_dims* dims, const moe_weights* w, const moe_experts_mx* mx, const uint16_t* gamma,
                      float eps, const uint16_t* x, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const BlockArgs blk{x, gamma, eps};
  return forward_impl(dims, w, nullptr, out, ws, ws_bytes, stream, Marks{nullptr, stream}, mx, &blk);
}

int moe_bias_update(const int32_t* offsets, int32_t E, float eta, float* corr_bias, hipStream_t stream) {
  if (offsets == nullptr || corr_bias == nullptr || E <= 0 || !(eta == eta) || eta > 1e30f || eta < -1e30f)
    return MOE_ERR_INVALID;
  return hip_status(launch_bias_update(offsets, E, eta, corr_bias, stream));
}

int moe_quantize_mxfp8(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                       hipStream_t stream) {
  if (rows <= 0 || cols <= 0 || cols % 32) return MOE_ERR_INVALID;
  if (src == nullptr || codes == nullptr || scales == nullptr) return MOE_ERR_INVALID;
  if (((uintptr_t)src | (uintptr_t)codes) & 15) return MOE_ERR_INVALID;
  return hip_status(launch_mxfp8_quantize(src, rows * (cols / 32), codes, scales, stream));
}

}  // extern "C"

namespace {

// Scratch of the allocation-free forward: a static device array (one copy per
// GPU, held until the process ends). In host code its name is only a stand-in;
// kernels take the device address looked up below.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The device address of the current device's copy of `scratch`, looked up on
// the first call on each device and kept; nullptr if the lookup fails.
void* scratch_for_current_device() {
  static std::mutex mu;
  static void* per_dev[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (per_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    per_dev[dev] = p;
  }
  return per_dev[dev];
}

}  // namespace

extern "C" {

int moe_forward_noalloc(const moe_dims* dims, const moe_weights* w, const uint16_t* x, uint16_t* out,
                        hipStream_t stream) {
  int st;
  if (!dims_ok(dims, &st)) return st;
  if (make_layout(*dims).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  void* ws = scratch_for_current_device();
  if (ws == nullptr) return MOE_ERR_HIP;
  return forward_impl(dims, w, x, out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, Marks{nullptr, stream});
}

}  // extern "C"
