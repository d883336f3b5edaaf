// kernels.h -- internal launchers of libmoe (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_MAX_EXPERTS 256
// picks per token of the pick-by-pick top-k (the small-batch routes); beyond
// it the top-k selects by ranks
#define MOE_MAX_TOPK 8
#define DISPATCH_RUN 512  // slots per histogram run

// grouped (prefill) GEMM tile: weight rows x token rows x K step
#define GG_BW 256
#define GG_BT 256
#ifndef GG_BK
#define GG_BK 64
#endif

struct RouterArgs {
  const void* x;          // [T][H] bf16 or fp32
  int T, H, E, k;
  int dtype_f32;
  const void* wr;         // [H][E]
  const float* bias;      // [E] or null
  const float* logits_in; // [T][E] or null
  int32_t* idx;           // [T][k]
  float* w;               // [T][k]
  float* part;            // [router_splits(T, H, E)][T][E] partial logits (bf16 layers)
  uint16_t* wrt;          // [E][H] workspace for the transposed router (bf16 layers)
  int raw_gate;           // 1: gate weights = the selected logits (no softmax)
  // residual layers on the one-workgroup small-batch route: the fp32 stream
  // [T][H], and the branch input [T][H] bf16 the route forms from it (x is
  // then not read)
  const float* hres = nullptr;
  uint16_t* xt_out = nullptr;
  // uint8 expert layers on that route: the expert input [T][H] as fp16 (the
  // route writes it; no separate conversion)
  uint16_t* x16_out = nullptr;
};

struct DispatchArgs {
  const int32_t* idx;  // [S]
  int S, E;
  int tile_rows;       // token rows per grouped-GEMM tile
  int32_t* hist;       // [nrun][E]
  int32_t* rank;       // [S]
  int32_t* base;       // [nrun][E]
  int32_t* counts;     // [E]
  int32_t* offsets;    // [E+1]
  int32_t* tile_off;   // [E+1]
  int32_t* active;     // [E+1]
  int32_t* perm;       // [S]
  int32_t* inv;        // [S]
  int capacity;        // pairs an expert keeps, 0 = all
  // the single-token route may leave the dispatch out (its outputs are then
  // not written): the expert kernels that follow take the slots in order
  bool none = false;
};

struct ExpertArgs {
  const void* x;            // [T][H] layer input (bf16 or fp32)
  const void* experts;      // expert blocks
  uint64_t stride_elems;    // expert stride in elements (bytes for uint8 experts)
  int u8;                   // experts are uint8 codes + parameter blocks; then x
                            // holds fp16 values and act is stored in fp16
  int T, H, F, E, k, S;
  int rows_hint;            // rows per expert one streaming pass should cover
  const int32_t* perm;      // [S]
  const int32_t* offsets;   // [E+1]
  const int32_t* tile_off;  // [E+1]
  const int32_t* active;    // [E+1]
  void* act;                // [S][F] bf16 or fp32
  float* yp;                // [S][H] fp32
  // grouped GEMMs: partial sums of split tail tiles, one 256 KB slot per
  // workgroup (grouped_grid() of them), or null (no split)
  float* gws = nullptr;
  // slot of each pair [T][k] (-1: dropped by the capacity; the
  // single-token kernels take null as slot j = row j, none dropped); step 5
  // inputs for a down projection that folds the combine in (cy null: it may
  // not): gate weights [T][k], residual [T][H] or null, output [T][H]
  const int32_t* cinv = nullptr;
  // the expert of each pair [T][k] (the single-token kernels read the
  // routing directly: slot j's weights and activation row in one step)
  const int32_t* cidx = nullptr;
  const float* cw = nullptr;
  const float* cres = nullptr;
  float* cy = nullptr;
};

int router_splits(int T, int H, int E);
int launch_router(const RouterArgs& a, hipStream_t st);
int launch_prenorm(const float* h, int T, int H, uint16_t* xt, hipStream_t st);
// bf16 routing + dispatch in one launch for T <= 64 (counter: zeroed int32,
// left zeroed by the kernel)
int launch_route_small(const RouterArgs& a, const DispatchArgs& d, int32_t* counter,
                       hipStream_t st);
// whether launch_route_small can form the prenorm branch input itself
bool route_small_folds_prenorm(int T, int H, int E);
// whether launch_route_small can write the fp16 copy of the expert input
bool route_small_writes_x16(int T, int H, int E);
int launch_dispatch(const DispatchArgs& a, hipStream_t st);

// compute units of the current device (cached per device)
int cu_count();

// bf16 expert FFN, grouped MFMA GEMMs (many rows per expert)
int launch_grouped_gate_up(const ExpertArgs& a, hipStream_t st);
// split-K factor the grouped down projection uses for this call (1 or 2);
// with 2 it writes two partial planes yp[2][S][H]
int grouped_down_ksplit(const ExpertArgs& a);
// workgroups of a grouped GEMM launch on the current device
int grouped_grid();
int launch_grouped_down(const ExpertArgs& a, int ksplit, hipStream_t st);
// bf16 expert FFN, weight-streaming MFMA kernels (few rows per expert; every
// batch for uint8 experts)
int launch_stream_gate_up(const ExpertArgs& a, hipStream_t st);
// *combined: set when the launch also wrote y (step 5 folded in)
int launch_stream_down(const ExpertArgs& a, bool* combined, hipStream_t st);
// fp32 expert FFN (plain FMA)
// single-token path (T == 1): the routed experts' weights streamed into
// registers, matrix-vector products on the dot instructions, the combine
// folded into the down projection when cy is set (then *combined = true)
bool gemv_supported(int T, int H, int F, int k, bool u8);
int launch_gemv_gate_up(const ExpertArgs& a, hipStream_t st);
int launch_gemv_down(const ExpertArgs& a, bool* combined, hipStream_t st);
int launch_f32_gate_up(const ExpertArgs& a, hipStream_t st);
int launch_f32_down(const ExpertArgs& a, hipStream_t st);

// fp16 copy of n bf16 values (exact in fp16's normal range; round toward
// zero beyond it and below it)
int launch_to_f16(const uint16_t* src, size_t n, uint16_t* dst, hipStream_t st);

// uint8 expert weights from bf16 ones (parameter blocks of dst as scratch)
int launch_quantize_u8(const void* src, uint64_t src_stride, int E, int H, int F, void* dst,
                       uint64_t dst_stride, hipStream_t st);

// y[t] = resid[t] + sum_j w[t][j] * (sum over planes q of yp[q][inv[t*k+j]])
int launch_combine(const float* yp, int nplanes, const float* w, const int32_t* inv,
                   const float* resid, int T, int H, int k, float* y, hipStream_t st);
