// moe_api.hip -- host side of the C ABI declared in include/moe.h.
//
// init / forward / free with caller-owned buffers follows the pages' C API
// [zskr.cn/news/2275853 "Colibri：面向MoE架构的C语言高效推理引擎解析" sec. 3.2
// and 4.2: buffers pre-allocated for a maximum size, explicit invalid-argument
// error codes; www.pnsm.cn/news/1892388.html sec. 2.1 and 4.4: init, forward,
// free].  The layer's device workspace is carved from one allocation by a
// bump ("arena") allocator with power-of-two alignment [www.pnsm.cn page
// sec. 3.2], sized once for max_tokens so no call allocates.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "kernels.h"
#include "moe.h"

struct moe_layer {
  moe_layer_desc d;
  int device;
  size_t esize;
  void* ws;
  size_t ws_bytes;
  // workspace pieces
  uint16_t* xt;       // [maxT][H] bf16 branch input (RESIDUAL_PRENORM)
  uint16_t* x16;      // [maxT][H] fp16 copy of the expert input (uint8 experts)
  int32_t* idx;       // [S]
  float* w;           // [S]
  float* part;        // partial router logits
  uint16_t* wrt;      // [E][H] transposed router (bf16 layers)
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E+1]
  int32_t* tile_off;  // [E+1]
  int32_t* active;    // [E+1]
  int32_t* hist;      // [nrun][E]
  int32_t* base;      // [nrun][E]
  int32_t* rank;      // [S]
  int32_t* perm;      // [S]
  int32_t* inv;       // [S]
  void* act;          // [S][F] dtype
  float* yp;          // [2][S][H]
  int32_t* sync;      // [1] zeroed completion counter of the fused small-batch router
  int gslots;         // workgroups of the grouped GEMMs (0: the layer never runs them)
  float* gws;         // [gslots][256 x 256] partial sums of split tail tiles
};

namespace {

constexpr uint32_t kKnownFlags = MOE_FLAG_RESIDUAL_PRENORM | MOE_FLAG_PATH_GROUPED |
                                 MOE_FLAG_PATH_STREAM | MOE_FLAG_GATE_RAW |
                                 MOE_FLAG_COMBINE_SEPARATE;

struct Arena {
  char* base;
  size_t cap;
  size_t off;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) & ~(a - 1); }

// Returns the next 256-byte aligned block of n bytes.  With base == nullptr
// it only measures (cap ignored).
void* arena_alloc(Arena& A, size_t n) {
  const size_t o = align_up(A.off, 256);
  A.off = o + n;
  if (!A.base) return nullptr;
  if (A.off > A.cap) return nullptr;
  return A.base + o;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int validate_desc(const moe_layer_desc* d) {
  if (!d || d->struct_size != sizeof(moe_layer_desc)) return MOE_ERR_INVALID_ARG;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d->hidden < 1 || d->ffn < 1 || d->num_experts < 1 || d->top_k < 1)
    return MOE_ERR_INVALID_ARG;
  if (d->top_k > d->num_experts) return MOE_ERR_INVALID_ARG;
  if (d->max_tokens < 1 || d->max_tokens > 65536) return MOE_ERR_INVALID_ARG;
  if (d->flags & ~kKnownFlags) return MOE_ERR_INVALID_ARG;
  if ((d->flags & MOE_FLAG_PATH_GROUPED) && (d->flags & MOE_FLAG_PATH_STREAM))
    return MOE_ERR_INVALID_ARG;
  if (!d->router_w || !d->expert_base) return MOE_ERR_INVALID_ARG;
  if (!aligned16(d->router_w) || !aligned16(d->expert_base)) return MOE_ERR_INVALID_ARG;
  if (d->router_b && ((uintptr_t)d->router_b & 3u)) return MOE_ERR_INVALID_ARG;
  const uint64_t es = d->dtype == MOE_F32 ? 4 : 2;
  const uint64_t H = (uint64_t)d->hidden, F = (uint64_t)d->ffn;
  if (d->expert_format != MOE_EXPERT_DTYPE && d->expert_format != MOE_EXPERT_U8)
    return MOE_ERR_INVALID_ARG;
  const bool u8 = d->expert_format == MOE_EXPERT_U8;
  const uint64_t need = u8 ? 3 * H * F + sizeof(moe_u8_params) : 3 * H * F * es;
  if (d->expert_stride < need || (d->expert_stride & 255u)) return MOE_ERR_INVALID_ARG;
  if (u8 && (d->dtype != MOE_BF16 || (d->flags & MOE_FLAG_PATH_GROUPED)))
    return MOE_ERR_UNSUPPORTED;
  if (d->num_experts > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (d->dtype == MOE_BF16 && (H % 256 || F % 128)) return MOE_ERR_UNSUPPORTED;
  if (d->dtype == MOE_F32 && (H % 4 || F % 4)) return MOE_ERR_UNSUPPORTED;
  if ((d->flags & MOE_FLAG_RESIDUAL_PRENORM) && (d->dtype != MOE_BF16 || H > 16384))
    return MOE_ERR_UNSUPPORTED;
  const uint64_t S = (uint64_t)d->max_tokens * (uint64_t)d->top_k;
  const uint64_t lim = 1ull << 31;
  if (S * (H > F ? H : F) >= lim || 3 * H * F >= lim || (uint64_t)d->max_tokens * H >= lim)
    return MOE_ERR_UNSUPPORTED;
  if (d->expert_capacity < 0) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// split_ws: also carve the grouped GEMMs' tail-split partial sums (64 MB on
// 256 CUs) when the layer runs them
void carve(moe_layer* L, Arena& A, bool split_ws = true) {
  const moe_layer_desc& d = L->d;
  const size_t S = (size_t)d.max_tokens * d.top_k;
  const size_t E = (size_t)d.num_experts;
  const size_t nrun = (S + DISPATCH_RUN - 1) / DISPATCH_RUN;
  L->xt = (uint16_t*)arena_alloc(A, (d.flags & MOE_FLAG_RESIDUAL_PRENORM)
                                        ? (size_t)d.max_tokens * d.hidden * 2 : 0);
  L->x16 = (uint16_t*)arena_alloc(A, d.expert_format == MOE_EXPERT_U8
                                         ? (size_t)d.max_tokens * d.hidden * 2 : 0);
  L->idx = (int32_t*)arena_alloc(A, S * 4);
  L->w = (float*)arena_alloc(A, S * 4);
  size_t part = 0;
  if (d.dtype == MOE_BF16) {
    for (int tiles = 1; (tiles - 1) * 64 < d.max_tokens; ++tiles) {
      const int T = tiles * 64 < d.max_tokens ? tiles * 64 : d.max_tokens;
      const size_t need = (size_t)router_splits(T, d.hidden, E) * T * E * 4;
      if (need > part) part = need;
    }
  }
  L->part = (float*)arena_alloc(A, part);
  L->wrt = (uint16_t*)arena_alloc(A, d.dtype == MOE_BF16 ? E * (size_t)d.hidden * 2 : 0);
  L->counts = (int32_t*)arena_alloc(A, E * 4);
  L->offsets = (int32_t*)arena_alloc(A, (E + 1) * 4);
  L->tile_off = (int32_t*)arena_alloc(A, (E + 1) * 4);
  L->active = (int32_t*)arena_alloc(A, (E + 1) * 4);
  L->hist = (int32_t*)arena_alloc(A, nrun * E * 4);
  L->base = (int32_t*)arena_alloc(A, nrun * E * 4);
  L->rank = (int32_t*)arena_alloc(A, S * 4);
  L->perm = (int32_t*)arena_alloc(A, S * 4);
  L->inv = (int32_t*)arena_alloc(A, S * 4);
  L->act = arena_alloc(A, S * (size_t)d.ffn * L->esize);
  // two planes: the grouped down projection may split its K range in two
  L->yp = (float*)arena_alloc(A, 2 * S * (size_t)d.hidden * 4);
  L->sync = (int32_t*)arena_alloc(A, 4);
  // the grouped GEMMs run when T * k > 32 * E (or when pinned to them)
  const bool grouped = split_ws && d.dtype == MOE_BF16 && d.expert_format != MOE_EXPERT_U8 &&
                       !(d.flags & MOE_FLAG_PATH_STREAM) &&
                       ((d.flags & MOE_FLAG_PATH_GROUPED) || S > 32 * E);
  L->gslots = grouped ? grouped_grid() : 0;
  L->gws = (float*)arena_alloc(A, (size_t)L->gslots * 256 * 256 * 4);
}

// Keeps the layer's device current for the duration of a call.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool use_stream_path(const moe_layer* L, int T) {
  if (L->d.expert_format == MOE_EXPERT_U8) return true;
  if (L->d.flags & MOE_FLAG_PATH_STREAM) return true;
  if (L->d.flags & MOE_FLAG_PATH_GROUPED) return false;
  // average rows per expert; the grouped GEMM works on 256-row tiles
  return (int64_t)T * L->d.top_k <= 32 * (int64_t)L->d.num_experts;
}

// Routing and dispatch in one launch (bf16 layers, one token tile, up to
// MOE_MAX_TOPK picks per token).
bool small_route(const moe_layer* L, int T, const float* logits_in) {
  return L->d.dtype == MOE_BF16 && !logits_in && T <= 64 && L->d.top_k <= MOE_MAX_TOPK;
}

// Steps 1-3 into the workspace.  x_route is the routing input (bf16 branch
// input or the layer input), or nullptr when logits_in is given.
int run_route(moe_layer* L, const void* x_route, int T, const float* logits_in,
              int tile_rows, hipStream_t st) {
  const moe_layer_desc& d = L->d;
  RouterArgs ra{x_route, T, d.hidden, d.num_experts, d.top_k, d.dtype == MOE_F32 ? 1 : 0,
                d.router_w, d.router_b, logits_in, L->idx, L->w, L->part, L->wrt,
                (d.flags & MOE_FLAG_GATE_RAW) ? 1 : 0};
  DispatchArgs da{L->idx, T * d.top_k, d.num_experts, tile_rows, L->hist, L->rank, L->base,
                  L->counts, L->offsets, L->tile_off, L->active, L->perm, L->inv,
                  d.expert_capacity};
  if (small_route(L, T, logits_in)) return launch_route_small(ra, da, L->sync, st) ? MOE_ERR_DEVICE : MOE_OK;
  if (launch_router(ra, st)) return MOE_ERR_DEVICE;
  if (launch_dispatch(da, st)) return MOE_ERR_DEVICE;
  return MOE_OK;
}

// ---- the entry point that allocates nothing (moe_forward_noalloc) ----------
//
// Its workspace is this file-scope array, one copy per GPU for the life of
// the process.  The first 256 bytes hold the small-batch route's completion
// counter (zero between calls: cleared once per device at set-up, and every
// route launch leaves it at zero); the workspace of a call is carved after
// them, sized for that call's T.
constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchHead = 256;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_i32_kernel(int32_t* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

std::mutex g_scratch_mu;
unsigned char* g_scratch[64];  // device address of `scratch` per device

// The device address of this device's scratch array (set-up on first use:
// the address, then a fill kernel on `st` that clears the counter).
unsigned char* scratch_base(int dev, hipStream_t st) {
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    zero_i32_kernel<<<1, 64, 0, st>>>((int32_t*)p, (int)(kScratchHead / 4));
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_scratch[dev] = (unsigned char*)p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

moe_layer_t* moe_layer_create(const moe_layer_desc* d, int* status) {
  int rc = validate_desc(d);
  if (rc != MOE_OK) {
    if (status) *status = rc;
    return nullptr;
  }
  moe_layer* L = (moe_layer*)calloc(1, sizeof(moe_layer));
  if (!L) {
    if (status) *status = MOE_ERR_NO_MEMORY;
    return nullptr;
  }
  L->d = *d;
  L->esize = d->dtype == MOE_F32 ? 4 : 2;
  if (hipGetDevice(&L->device) != hipSuccess) {
    free(L);
    if (status) *status = MOE_ERR_DEVICE;
    return nullptr;
  }
  Arena measure{nullptr, 0, 0};
  carve(L, measure);
  L->ws_bytes = align_up(measure.off, 256);
  if (hipMalloc(&L->ws, L->ws_bytes) != hipSuccess) {
    (void)hipGetLastError();
    free(L);
    if (status) *status = MOE_ERR_NO_MEMORY;
    return nullptr;
  }
  Arena real{(char*)L->ws, L->ws_bytes, 0};
  carve(L, real);
  // the fused router's completion counter starts at zero and every launch
  // leaves it at zero
  if (hipMemset(L->sync, 0, 4) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(L->ws);
    free(L);
    if (status) *status = MOE_ERR_DEVICE;
    return nullptr;
  }
  if (status) *status = MOE_OK;
  return L;
}

int moe_route(moe_layer_t* L, const void* x, int32_t T, const float* logits_in,
              int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
              int32_t* perm, int32_t* inv, void* stream) {
  if (!L) return MOE_ERR_INVALID_ARG;
  const moe_layer_desc& d = L->d;
  if (T < 1 || T > d.max_tokens) return MOE_ERR_INVALID_ARG;
  if (!logits_in && (!x || !aligned16(x))) return MOE_ERR_INVALID_ARG;
  if (logits_in && !aligned16(logits_in)) return MOE_ERR_INVALID_ARG;
  if (!topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  DeviceGuard g(L->device);
  if (!g.ok) return MOE_ERR_DEVICE;
  hipStream_t st = (hipStream_t)stream;
  const int S = T * d.top_k;
  const void* xr = x;
  if (!logits_in && (d.flags & MOE_FLAG_RESIDUAL_PRENORM)) {
    if (launch_prenorm((const float*)x, T, d.hidden, L->xt, st)) return MOE_ERR_DEVICE;
    xr = L->xt;
  }
  int rc = run_route(L, logits_in ? nullptr : xr, T, logits_in, GG_BT, st);
  if (rc) return rc;
  const size_t E = (size_t)d.num_experts;
  hipError_t e = hipSuccess;
  auto cp = [&](void* dst, const void* src, size_t n) {
    if (dst && e == hipSuccess) e = hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, st);
  };
  cp(topk_idx, L->idx, (size_t)S * 4);
  cp(topk_w, L->w, (size_t)S * 4);
  cp(counts, L->counts, E * 4);
  cp(offsets, L->offsets, (E + 1) * 4);
  cp(perm, L->perm, (size_t)S * 4);
  cp(inv, L->inv, (size_t)S * 4);
  return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

int moe_forward(moe_layer_t* L, const void* x, int32_t T, float* y, void* stream) {
  return moe_forward_ev(L, x, T, y, stream, nullptr);
}

int moe_forward_ev(moe_layer_t* L, const void* x, int32_t T, float* y, void* stream,
                   void* const* stage_events) {
  if (!L) return MOE_ERR_INVALID_ARG;
  const moe_layer_desc& d = L->d;
  if (T < 1 || T > d.max_tokens) return MOE_ERR_INVALID_ARG;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  const bool prenorm = (d.flags & MOE_FLAG_RESIDUAL_PRENORM) != 0;
  const size_t xbytes = (size_t)T * d.hidden * (prenorm ? 4 : L->esize);
  const size_t ybytes = (size_t)T * d.hidden * 4;
  if (prenorm) {
    if (x != (const void*)y && ranges_overlap(x, xbytes, y, ybytes)) return MOE_ERR_INVALID_ARG;
  } else if (ranges_overlap(x, xbytes, y, ybytes)) {
    return MOE_ERR_INVALID_ARG;
  }
  DeviceGuard g(L->device);
  if (!g.ok) return MOE_ERR_DEVICE;
  hipStream_t st = (hipStream_t)stream;
  auto mark = [&](int i) -> bool {
    return !stage_events || hipEventRecord((hipEvent_t)stage_events[i], st) == hipSuccess;
  };
  const int S = T * d.top_k;
  const void* xin = x;
  if (!mark(MOE_STAGE_ROUTE)) return MOE_ERR_DEVICE;
  // residual layers: the small-batch route forms the branch input itself
  // when it runs in one workgroup per 16 tokens; otherwise a kernel of its own
  const bool fold_pn = prenorm && small_route(L, T, nullptr) &&
                       route_small_folds_prenorm(T, d.hidden, d.num_experts);
  // uint8 layers: the same route writes the fp16 expert input
  const bool fold_x16 = d.expert_format == MOE_EXPERT_U8 && small_route(L, T, nullptr) &&
                        route_small_writes_x16(T, d.hidden, d.num_experts);
  if (prenorm) {
    if (!fold_pn && launch_prenorm((const float*)x, T, d.hidden, L->xt, st))
      return MOE_ERR_DEVICE;
    xin = L->xt;
  }
  const bool f32 = d.dtype == MOE_F32;
  const bool stream_path = !f32 && use_stream_path(L, T);
  // a single token: matrix-vector kernels (unless the streaming kernels are
  // asked for by flag)
  const bool gemv_path = stream_path && !(d.flags & MOE_FLAG_PATH_STREAM) &&
                         gemv_supported(T, d.hidden, d.ffn, d.top_k,
                                        d.expert_format == MOE_EXPERT_U8);
  const bool slot_order = gemv_path && !(d.flags & MOE_FLAG_COMBINE_SEPARATE);
  {
    const moe_layer_desc& dd = L->d;
    RouterArgs ra{xin, T, dd.hidden, dd.num_experts, dd.top_k, f32 ? 1 : 0, dd.router_w,
                  dd.router_b, nullptr, L->idx, L->w, L->part, L->wrt,
                  (dd.flags & MOE_FLAG_GATE_RAW) ? 1 : 0};
    DispatchArgs da{L->idx, S, dd.num_experts, GG_BT, L->hist, L->rank, L->base, L->counts,
                    L->offsets, L->tile_off, L->active, L->perm, L->inv, dd.expert_capacity};
    // a single token on the matrix-vector kernels with the combine folded
    // in: its activation rows in slot order, no dispatch (no pair of one
    // token is ever dropped)
    da.none = slot_order;
    if (fold_pn) {
      ra.hres = (const float*)x;
      ra.xt_out = L->xt;
    }
    if (fold_x16) ra.x16_out = L->x16;
    if (small_route(L, T, nullptr)) {  // one launch: the dispatch stage is empty
      if (launch_route_small(ra, da, L->sync, st)) return MOE_ERR_DEVICE;
      if (!mark(MOE_STAGE_DISPATCH)) return MOE_ERR_DEVICE;
    } else {
      if (launch_router(ra, st)) return MOE_ERR_DEVICE;
      if (!mark(MOE_STAGE_DISPATCH)) return MOE_ERR_DEVICE;
      if (launch_dispatch(da, st)) return MOE_ERR_DEVICE;
    }
  }
  ExpertArgs ea{};
  ea.x = xin;
  ea.experts = d.expert_base;
  ea.u8 = d.expert_format == MOE_EXPERT_U8;
  ea.stride_elems = ea.u8 ? d.expert_stride : d.expert_stride / L->esize;
  ea.T = T;
  ea.H = d.hidden;
  ea.F = d.ffn;
  ea.E = d.num_experts;
  ea.k = d.top_k;
  ea.S = S;
  ea.perm = L->perm;
  ea.offsets = L->offsets;
  ea.tile_off = L->tile_off;
  ea.active = L->active;
  ea.act = L->act;
  ea.yp = L->yp;
  if (L->gslots > 0 && L->gslots == grouped_grid()) ea.gws = L->gws;
  {
    // rows an expert is expected to see, for the width of a streaming pass
    const int avg = (S + d.num_experts - 1) / d.num_experts;
    int hint = 2 * avg < 16 ? 16 : 2 * avg;
    ea.rows_hint = T < hint ? T : hint;
  }
  // the single-token kernels find each slot's expert and rows through these
  ea.cinv = slot_order ? nullptr : L->inv;
  ea.cidx = L->idx;
  if (!mark(MOE_STAGE_GATE_UP)) return MOE_ERR_DEVICE;
  if (ea.u8) {  // the uint8 kernels take fp16 token operands
    if (!fold_x16 &&
        launch_to_f16((const uint16_t*)xin, (size_t)T * d.hidden, L->x16, st))
      return MOE_ERR_DEVICE;
    ea.x = L->x16;
  }
  int r1 = f32           ? launch_f32_gate_up(ea, st)
           : gemv_path   ? launch_gemv_gate_up(ea, st)
           : stream_path ? launch_stream_gate_up(ea, st)
                         : launch_grouped_gate_up(ea, st);
  if (r1 || !mark(MOE_STAGE_DOWN)) return MOE_ERR_DEVICE;
  const float* resid = prenorm ? (const float*)x : nullptr;
  const int planes = (f32 || stream_path) ? 1 : grouped_down_ksplit(ea);
  // the streaming down projection may take step 5 over (then the combine
  // stage below is empty)
  bool combined = false;
  if (stream_path && !(d.flags & MOE_FLAG_COMBINE_SEPARATE)) {
    ea.cw = L->w;
    ea.cres = resid;
    ea.cy = (float*)y;
  }
  int r2 = f32           ? launch_f32_down(ea, st)
           : gemv_path   ? launch_gemv_down(ea, &combined, st)
           : stream_path ? launch_stream_down(ea, &combined, st)
                         : launch_grouped_down(ea, planes, st);
  if (r2 || !mark(MOE_STAGE_COMBINE)) return MOE_ERR_DEVICE;
  if (!combined &&
      launch_combine(L->yp, planes, L->w, L->inv, resid, T, d.hidden, d.top_k, y, st))
    return MOE_ERR_DEVICE;
  if (!mark(MOE_NUM_STAGES)) return MOE_ERR_DEVICE;
  return MOE_OK;
}

int moe_forward_noalloc(const moe_layer_desc* d, const void* x, int32_t T, float* y,
                        void* stream) {
  int rc = validate_desc(d);
  if (rc != MOE_OK) return rc;
  if (T < 1 || T > d->max_tokens) return MOE_ERR_INVALID_ARG;
  // a layer on the host stack whose workspace is carved from the scratch
  // array for this call's T (no tail-split partial sums: they would take the
  // whole array)
  moe_layer L;
  memset(&L, 0, sizeof L);
  L.d = *d;
  L.d.max_tokens = T;
  L.esize = d->dtype == MOE_F32 ? 4 : 2;
  Arena measure{nullptr, 0, 0};
  carve(&L, measure, false);
  if (align_up(measure.off, 256) > kScratchBytes - kScratchHead) return MOE_ERR_UNSUPPORTED;
  if (hipGetDevice(&L.device) != hipSuccess) return MOE_ERR_DEVICE;
  unsigned char* base = scratch_base(L.device, (hipStream_t)stream);
  if (!base) return MOE_ERR_DEVICE;
  Arena real{(char*)base + kScratchHead, kScratchBytes - kScratchHead, 0};
  carve(&L, real, false);
  L.sync = (int32_t*)base;
  L.gslots = 0;
  L.gws = nullptr;
  return moe_forward_ev(&L, x, T, y, stream, nullptr);
}

void moe_layer_free(moe_layer_t* L) {
  if (!L) return;
  {
    DeviceGuard g(L->device);
    if (L->ws) (void)hipFree(L->ws);
  }
  free(L);
}

int moe_quantize_experts_u8(const void* src, uint64_t src_stride, int32_t E, int32_t H,
                            int32_t F, void* dst, uint64_t dst_stride, void* stream) {
  static_assert(sizeof(moe_u8_params) == 64, "parameter block");
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return MOE_ERR_INVALID_ARG;
  if (E < 1 || H < 1 || F < 1 || H % 16 || F % 16) return MOE_ERR_INVALID_ARG;
  const uint64_t hf = (uint64_t)H * (uint64_t)F;
  if (3 * hf >= (1ull << 31)) return MOE_ERR_INVALID_ARG;
  if (src_stride < 6 * hf || dst_stride < 3 * hf + sizeof(moe_u8_params) || (src_stride & 255u) ||
      (dst_stride & 255u))
    return MOE_ERR_INVALID_ARG;
  const uint64_t ns = (uint64_t)(E - 1) * src_stride + 6 * hf;
  const uint64_t nd = (uint64_t)(E - 1) * dst_stride + 3 * hf + sizeof(moe_u8_params);
  if (ranges_overlap(src, ns, dst, nd)) return MOE_ERR_INVALID_ARG;
  if (launch_quantize_u8(src, src_stride, E, H, F, dst, dst_stride, (hipStream_t)stream))
    return MOE_ERR_DEVICE;
  return MOE_OK;
}

}  // extern "C"
