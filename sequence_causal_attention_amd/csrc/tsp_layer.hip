// tsp_layer.hip -- C ABI of the bf16 projection GEMM and of one rank's TSP attention layer
// forward (gfx950): argument validation, tile configuration, and the schedule over the
// weight shards. The operations and their arguments are documented in tsp_attn.h.
#include <hip/hip_runtime.h>

#include "tsp_attn.h"
#include "attn_common.h"
#include "gemm_bf16.h"
#include "host_common.h"

namespace {

using tsp_host::aligned16;
using tsp_host::fail;

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

template <int BM, int BN, int WM, int WN>
hipError_t gemm_enqueue(tsp::GemmParams gp, hipStream_t stream) {
  gp.n_tiles_m = (gp.M + BM - 1) / BM;
  gp.n_tiles_n = (gp.N + BN - 1) / BN;
  const int64_t tiles = (int64_t)gp.n_tiles_m * gp.n_tiles_n;
  (void)hipGetLastError();
  hipLaunchKernelGGL((tsp::gemm_nt_bf16_kernel<BM, BN, WM, WN>), dim3((unsigned)tiles), dim3(WM * WN * 64), 0,
                     stream, gp);
  return hipGetLastError();
}

// Validates and launches one GEMM. gp.seg[0 .. nseg) must be filled in (their c, ldc,
// n_end, b_row, zigzag), and the zigzag fields when a segment uses the row map.
int gemm_launch(const char* what, tsp::GemmParams gp, hipStream_t stream) {
  if (!gp.a || !gp.b || (gp.mode == tsp::GEMM_ADD_F32_TO_BF16 && !gp.c2))
    return fail(TSP_EINVAL, "%s: null pointer argument", what);
  if (gp.nseg < 1 || gp.nseg > tsp::GEMM_MAX_SEG) return fail(TSP_EINVAL, "%s: 1 to 3 column segments", what);
  if (gp.mode == tsp::GEMM_ADD_F32_TO_BF16 && gp.nseg != 1)
    return fail(TSP_EINVAL, "%s: the bf16 copy of an fp32 sum takes one segment", what);
  if (!aligned16(gp.a) || !aligned16(gp.b) || (gp.c2 && !aligned16(gp.c2)))
    return fail(TSP_EINVAL, "%s: pointers must be 16-byte aligned", what);
  if (gp.M < 1 || gp.N < 1 || gp.K < 1) return fail(TSP_EINVAL, "%s: M, N and K must be >= 1", what);
  if (gp.K % tsp::GEMM_BK != 0) return fail(TSP_EINVAL, "%s: K must be a multiple of %d", what, tsp::GEMM_BK);
  if (gp.lda < gp.K || gp.ldb < gp.K) return fail(TSP_EINVAL, "%s: leading dimensions of A / B too small", what);
  if (gp.lda % 8 != 0 || gp.ldb % 8 != 0) return fail(TSP_EINVAL, "%s: lda and ldb must be multiples of 8", what);
  if (gp.lda > (int64_t(1) << 22) || gp.ldb > (int64_t(1) << 22))
    return fail(TSP_EINVAL, "%s: lda / ldb above 2^22", what);
  bool zz = false;
  int32_t start = 0;
  int64_t b_first = 0, b_last = 0;
  for (int s = 0; s < gp.nseg; ++s) {
    const tsp::GemmSeg& sg = gp.seg[s];
    if (!sg.c) return fail(TSP_EINVAL, "%s: null pointer argument", what);
    if (!aligned16(sg.c)) return fail(TSP_EINVAL, "%s: pointers must be 16-byte aligned", what);
    const int32_t width = sg.n_end - start;
    if (width < 4 || width % 4 != 0 || sg.ldc % 4 != 0 || sg.ldc < width)
      return fail(TSP_EINVAL, "%s: column segments and row strides must be multiples of 4 (and fit)", what);
    if (sg.b_row < 0 || (s > 0 && sg.b_row < b_last)) return fail(TSP_EINVAL, "%s: B rows of the segments must ascend", what);
    if (s == 0) b_first = sg.b_row;
    b_last = (int64_t)sg.b_row + width;
    zz = zz || sg.zigzag;
    start = sg.n_end;
  }
  if (start != gp.N) return fail(TSP_EINVAL, "%s: the segments must cover the N columns", what);
  // per-lane 32-bit byte offsets: a tile's B rows span at most the segments' B rows
  if (gp.nseg > 1 && (b_last - b_first) * gp.ldb * 2 >= (int64_t(1) << 32))
    return fail(TSP_EINVAL, "%s: B rows of the segments span more than 4 GiB", what);
  if (!zz) gp.S_local = 0;
  const int64_t big = ((int64_t)(gp.M + 255) / 256) * ((gp.N + 255) / 256);
  const int64_t small = ((int64_t)(gp.M + 127) / 128) * ((gp.N + 127) / 128);
  if (small > 0x7fffffff) return fail(TSP_EINVAL, "%s: problem too large", what);
  const hipError_t e = big >= device_cus() ? gemm_enqueue<256, 256, 2, 4>(gp, stream)
                                           : gemm_enqueue<128, 128, 2, 2>(gp, stream);
  if (e != hipSuccess) return fail(TSP_ELAUNCH, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return TSP_OK;
}

// Workspace of the attention layer for groups of G weight shards, in bytes, each piece
// 256-byte aligned: the group's Q and attention output (bf16), its lse, and the fp32 sum of
// the output projection over the groups.
struct LayerWorkspace {
  int64_t q, o, lse, y, total;
};
LayerWorkspace layer_workspace(int64_t B, int64_t S_total, int64_t D, int64_t Hq, int64_t dh, int64_t d_model,
                               int64_t G) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t rows = B * (S_total / D);  // B * 2C local tokens
  const int64_t hg = G * (Hq / D);         // query heads of a group
  LayerWorkspace w{};
  w.q = 0;
  w.o = up(rows * hg * dh * 2);
  w.lse = w.o + up(rows * hg * dh * 2);
  w.y = w.lse + up(rows * hg * 4);
  w.total = w.y + up(rows * d_model * 4);
  return w;
}

int layer_check(int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh,
                int64_t d_model, int64_t G) {
  int st = tsp_host::check_sizes(S_total, D, rank);
  if (st != TSP_OK) return st;
  if (B < 1 || Hq < 1 || Hkv < 1 || d_model < 1) return fail(TSP_EINVAL, "B, heads and d_model must be >= 1");
  if (dh != 64 && dh != 128 && dh != 256) return fail(TSP_EUNSUPPORTED, "head dim %lld not in {64, 128, 256}", (long long)dh);
  if (Hq % Hkv != 0) return fail(TSP_EINVAL, "Hq not divisible by Hkv");
  if (Hq % D != 0 || Hkv % D != 0)
    return fail(TSP_EINVAL, "the weight shards split the heads: Hq and Hkv must be divisible by D");
  if (d_model % 64 != 0) return fail(TSP_EINVAL, "d_model must be a multiple of 64");
  if (d_model > (int64_t(1) << 22) || Hq * dh > (int64_t(1) << 22) || (Hq + 2 * Hkv) * dh > (int64_t(1) << 22))
    return fail(TSP_EINVAL, "layer too wide");
  if (B * (S_total / D) > 0x7fffffff) return fail(TSP_EINVAL, "too many local tokens");
  if (G < 0 || (G > 0 && D % G != 0))
    return fail(TSP_EINVAL, "shards_per_group must divide D (or be 0 for automatic)");
  return TSP_OK;
}

// Shards per group chosen automatically: the fewest whose attention launch has at least as
// many workgroups as the device has CUs (else all D).
int64_t auto_group(int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh) {
  const int cus = device_cus();
  for (int64_t G = 1; G < D; ++G) {
    if (D % G != 0) continue;
    TspParams ap{};
    if (tsp_host::attn_plan(B, S_total, D, rank, G * (Hq / D), G * (Hkv / D), dh, TSP_BF16, &ap) == TSP_OK &&
        ap.n_units >= cus)
      return G;
  }
  return D;
}

}  // namespace

extern "C" {

int tsp_gemm_bf16_nt(const void* a, const void* b, void* c, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                     int64_t ldc, int mode, void* stream) {
  if (mode != tsp::GEMM_STORE_BF16 && mode != tsp::GEMM_STORE_F32 && mode != tsp::GEMM_ADD_F32)
    return fail(TSP_EINVAL, "gemm: mode must be 0 (bf16), 1 (fp32) or 2 (fp32, accumulate)");
  if (M > 0x7fffffff || N > 0x7fffffff || K > 0x7fffffff || M < 1 || N < 1 || K < 1)
    return fail(TSP_EINVAL, "gemm: sizes must be in [1, 2^31)");
  tsp::GemmParams gp{};
  gp.a = static_cast<const uint16_t*>(a);
  gp.b = static_cast<const uint16_t*>(b);
  gp.lda = lda;
  gp.ldb = ldb;
  gp.M = (int32_t)M;
  gp.N = (int32_t)N;
  gp.K = (int32_t)K;
  gp.mode = mode;
  gp.nseg = 1;
  gp.seg[0].c = c;
  gp.seg[0].ldc = ldc;
  gp.seg[0].n_end = (int32_t)N;
  int st = gemm_launch("gemm", gp, static_cast<hipStream_t>(stream));
  return st == TSP_OK ? tsp_host::ok() : st;
}

int tsp_attn_layer_workspace_bytes(int64_t B, int64_t S_total, int64_t D, int64_t Hq, int64_t Hkv, int64_t dh,
                                   int64_t d_model, int64_t shards_per_group, int64_t* bytes) {
  if (!bytes) return fail(TSP_EINVAL, "null output pointer");
  int st = layer_check(B, S_total, D, 0, Hq, Hkv, dh, d_model, shards_per_group);
  if (st != TSP_OK) return st;
  *bytes = layer_workspace(B, S_total, D, Hq, dh, d_model, shards_per_group == 0 ? D : shards_per_group).total;
  return tsp_host::ok();
}

int tsp_attn_layer_fwd(const void* x_local, const void* w_qkv, const void* w_o, void* k_gathered, void* v_gathered,
                       void* y_local, void* workspace, int64_t workspace_bytes, int64_t B, int64_t S_total,
                       int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh, int64_t d_model,
                       int64_t shards_per_group, void* stream) {
  const void* ptrs[] = {x_local, w_qkv, w_o, k_gathered, v_gathered, y_local, workspace};
  for (const void* ptr : ptrs) {
    if (!ptr) return fail(TSP_EINVAL, "null pointer argument");
    if (!aligned16(ptr)) return fail(TSP_EINVAL, "pointers must be 16-byte aligned");
  }
  int st = layer_check(B, S_total, D, rank, Hq, Hkv, dh, d_model, shards_per_group);
  if (st != TSP_OK) return st;
  const int64_t G = shards_per_group > 0 ? shards_per_group : auto_group(B, S_total, D, rank, Hq, Hkv, dh);
  const LayerWorkspace ws = layer_workspace(B, S_total, D, Hq, dh, d_model, G);
  if (workspace_bytes < ws.total)
    return fail(TSP_EINVAL, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes, (long long)ws.total);
  const int64_t hs = Hq / D, hks = Hkv / D;  // heads of one weight shard
  const int64_t hg = G * hs, hkg = G * hks;  // ... of a group of G shards
  const int64_t n_groups = D / G;
  const int64_t rows = B * (S_total / D);
  uint8_t* wsp = static_cast<uint8_t*>(workspace);
  uint16_t* q_ws = reinterpret_cast<uint16_t*>(wsp + ws.q);
  uint16_t* o_ws = reinterpret_cast<uint16_t*>(wsp + ws.o);
  float* lse_ws = reinterpret_cast<float*>(wsp + ws.lse);
  float* y_acc = reinterpret_cast<float*>(wsp + ws.y);
  const uint16_t* x = static_cast<const uint16_t*>(x_local);
  const uint16_t* wqkv = static_cast<const uint16_t*>(w_qkv);
  const uint16_t* wo = static_cast<const uint16_t*>(w_o);
  uint16_t* kg = static_cast<uint16_t*>(k_gathered);
  uint16_t* vg = static_cast<uint16_t*>(v_gathered);
  hipStream_t s = static_cast<hipStream_t>(stream);

  // attention of one group's heads: q_ws against the gathered K/V of its KV heads
  TspParams ap{};
  if ((st = tsp_host::attn_plan(B, S_total, D, rank, hg, hkg, dh, TSP_BF16, &ap)) != TSP_OK) return st;
  ap.kv_stride = Hkv * dh;

  for (int64_t g = 0; g < n_groups; ++g) {  // groups of weight shards, in broadcast order
    const int64_t i0 = g * G;               // the group's first shard
    // one GEMM for the group's Q, K and V: three column segments of the packed weight rows
    tsp::GemmParams p{};
    p.a = x;
    p.lda = d_model;
    p.b = wqkv;
    p.ldb = d_model;
    p.M = (int32_t)rows;
    p.K = (int32_t)d_model;
    p.N = (int32_t)((hg + 2 * hkg) * dh);
    p.mode = tsp::GEMM_STORE_BF16;
    p.nseg = 3;
    p.S_total = (int32_t)S_total;
    p.C = (int32_t)(S_total / (2 * D));
    p.D = (int32_t)D;
    p.rank = (int32_t)rank;
    p.S_local = (int32_t)(S_total / D);
    // Q of the group's query heads: [rows, hg * dh], the attention's q_local
    p.seg[0] = tsp::GemmSeg{q_ws, hg * dh, (int32_t)(hg * dh), (int32_t)(i0 * hs * dh), 0, 0};
    // K and V of its KV heads, written at the tokens' global positions
    p.seg[1] = tsp::GemmSeg{kg + i0 * hks * dh, Hkv * dh, (int32_t)((hg + hkg) * dh),
                            (int32_t)((Hq + i0 * hks) * dh), 1, 0};
    p.seg[2] = tsp::GemmSeg{vg + i0 * hks * dh, Hkv * dh, (int32_t)((hg + 2 * hkg) * dh),
                            (int32_t)((Hq + Hkv + i0 * hks) * dh), 1, 0};
    if ((st = gemm_launch("layer qkv projection", p, s)) != TSP_OK) return st;
    // causal attention of the group's heads over the gathered K/V
    ap.q = q_ws;
    ap.k = kg + i0 * hks * dh;
    ap.v = vg + i0 * hks * dh;
    ap.out = o_ws;
    ap.lse = lse_ws;
    if ((st = tsp_host::attn_launch(ap, dh, TSP_BF16, s)) != TSP_OK) return st;
    // output projection of the group's heads, accumulated over the groups
    tsp::GemmParams po{};
    po.a = o_ws;
    po.lda = hg * dh;
    po.b = wo + i0 * hs * dh;
    po.ldb = Hq * dh;
    po.M = (int32_t)rows;
    po.K = (int32_t)(hg * dh);
    po.N = (int32_t)d_model;
    po.nseg = 1;
    if (n_groups == 1) {
      po.seg[0] = tsp::GemmSeg{y_local, d_model, (int32_t)d_model, 0, 0, 0};
      po.mode = tsp::GEMM_STORE_BF16;
    } else {
      po.seg[0] = tsp::GemmSeg{y_acc, d_model, (int32_t)d_model, 0, 0, 0};
      po.c2 = y_local;
      po.mode = g == 0 ? tsp::GEMM_STORE_F32 : (g == n_groups - 1 ? tsp::GEMM_ADD_F32_TO_BF16 : tsp::GEMM_ADD_F32);
    }
    if ((st = gemm_launch("layer output projection", po, s)) != TSP_OK) return st;
  }
  return tsp_host::ok();
}

}  // extern "C"
