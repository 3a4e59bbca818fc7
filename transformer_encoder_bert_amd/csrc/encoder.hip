// The C ABI of ftx: encoder handle, weight repacking, the per-layer launch sequence, and
// the step-level entry points.  Host code; every computation happens in the kernels of
// gemm.hip, attention.hip and elementwise.hip.
//
// Source: the Faster Transformer article (cloud.tencent.com/developer/article/1490359),
// section "什么是 Faster Transformer" (an encoder created for head count, size per head,
// batch size and maximum sentence length, FP16/FP32 modes, a C++ API) and section
// "Faster Transformer 优化原理" (one layer = matrix multiplies plus a few fused custom
// kernels; launch configuration chosen per shape).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "ftx.h"
#include "ftx_steps.h"
#include "abi_common.h"
#include "launch.h"

using namespace ftx;

std::string& ftx::last_error_slot() {
  thread_local std::string msg;
  return msg;
}

// Shape checks shared by create and the step entry points.  The encoder takes any sequence
// length up to FTX_MAX_SEQ_LEN (it pads internally to a multiple of 32); the step entry
// points work on the padded layout and need the multiple of 32.
ftx_status ftx::check_shape(int B, int S, int nh, int d, bool any_len) {
  if (B < 1 || S < 1 || nh < 1 || d < 1) return fail(FTX_ERR_INVALID_ARG, "shape values must be >= 1");
  if (d != 32 && d != 64) return fail(FTX_ERR_UNSUPPORTED, "size_per_head must be 32 or 64");
  if (S > FTX_MAX_SEQ_LEN) return fail(FTX_ERR_UNSUPPORTED, "seq_len above 512");
  if (!any_len && S % 32 != 0)
    return fail(FTX_ERR_UNSUPPORTED, "the step entry points need seq_len a multiple of 32");
  S = (S + 31) / 32 * 32;
  if ((long)nh * d > FTX_MAX_HIDDEN) return fail(FTX_ERR_UNSUPPORTED, "hidden size above 4096");
  // 32-bit element indices inside kernels: the largest tensor is [B*S][4H]
  if ((long long)B * S * 4 * nh * d >= (1LL << 31))
    return fail(FTX_ERR_UNSUPPORTED, "batch * seq_len * 4 * hidden must stay below 2^31");
  return FTX_OK;
}

namespace {

// Largest FFN intermediate (rows x F) the folded path keeps in one piece: two thirds of the
// 256 MB last-level cache, which then also holds the chunk's other operands.  (96 MB measured
// worse: BERT-large S512 B32 then runs FFN-out on 8192-row chunks, 11.72 -> 12.56 ms, and
// BERT-base B512 does not change.)
constexpr size_t kFfnChunkBytes = (size_t)160 << 20;

struct LayerW {
  void* w_qkv_t;  // [3H][H]
  void* b_qkv;    // [3H]
  void* w_qkvh_t; // [3H][H] rows ordered per head (Q_h, K_h, V_h), or null (fused attention)
  void* b_qkvh;   // [3H] in the same order
  void* w_o_t;    // [H][H]
  void* b_o;
  void* ln1_g;
  void* ln1_b;
  void* w1_t;     // [F][H]
  void* b1;       // [F]
  void* w2_t;     // [H][F]
  void* b2;
  void* ln2_g;
  void* ln2_b;
  // the first LayerNorm folded into the first FFN projection (null when the shape does not
  // allow it): W1^T with its columns scaled by ln1 gamma, the fp32 column sums of that
  // matrix and the fp32 bias b1 + beta W1
  void* w1g_t = nullptr;  // [F][H]
  float* c1 = nullptr;    // [F]
  float* b1f = nullptr;   // [F]
};

// Views of the forward's intermediate tensors, all carved from one block of device memory:
// the handle's own workspace (ftx_forward) or the library's static scratch
// (ftx_forward_static_workspace).
struct Workspace {
  void *q, *k, *vt, *ctx, *abuf, *y1, *u;
  void *xpad = nullptr, *spad = nullptr;  // [B][S][H] input copy and layer state when Sv < S
  float* y1f = nullptr;     // fp32 copy of Y1, the residual of the second LayerNorm (bf16 only)
  float* st1 = nullptr;     // [T][ntn] (mean, M2) pairs of Z1 per projection tile (folded LN1)
  float* splitk = nullptr;  // fp32 partial products of split-K projections
  size_t splitk_elems = 0;
};

}  // namespace

struct ftx_encoder {
  int B, S, nh, d, L, H, F, T;  // S: internal (padded) length, a multiple of 32; T = B S
  int Sv;                       // the caller's sequence length (S rounded up to 32 = S)
  ftx_dtype dt;
  size_t es;
  int device;
  DeviceInfo dev;  // CU and XCD counts, read at create
  void* weights = nullptr;
  void* ws_mem = nullptr;  // the workspace allocation
  size_t ws_bytes = 0;     // its size (the layout of layout_workspace)
  size_t splitk_need = 0;  // fp32 elements of split-K partials the plans use
  Workspace w;             // views into ws_mem
  std::vector<LayerW> layers;
  std::vector<char> ready;
  int fused = 1;
  int fused_attention = 1;  // 0 off, 1 from 256 rows and 64 tiles, 2 whenever the shape fits
  bool attn_fits = false;   // the per-head weight copy exists (16-bit, S = 32, d = 64)
  bool attn_out = false;    // small batch at S = 32: the attention also yields the
                            // attention-output projection's partials, split by head
  bool fold_fits = false;   // the first LayerNorm can fold into the first FFN projection
  int fold = 1;             // FTX_OPT_FOLD_LAYERNORM
  int ln1_bn = 0, ln1_ntn = 0;  // attention-output tile width and tiles per row (fold)
  int ffn_rows = 0;             // rows per FFN chunk on the folded path (T: one chunk)
  bool w2_prefetch_fits = false;  // FFN-out on 128x128 tiles, more tiles than CUs (folded path)
  int prefetch = 1;             // FTX_OPT_PREFETCH_WEIGHTS
  int timing = 0;
  int graph_mode = 0;
  // graph of one whole forward, captured for the (input, seq_lens, output) it was made with
  hipStream_t cap_stream = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t graph_exec = nullptr;
  const void* g_in = nullptr;
  const int32_t* g_lens = nullptr;
  void* g_out = nullptr;
  struct Mark {
    hipEvent_t start, stop;
    int step;
  };
  std::vector<Mark> marks;      // recorded, not yet read
  std::vector<hipEvent_t> pool; // free events
};

namespace {

ftx_status take_event(ftx_encoder* e, hipEvent_t* ev) {
  if (!e->pool.empty()) {
    *ev = e->pool.back();
    e->pool.pop_back();
    return FTX_OK;
  }
  FTX_HIP(hipEventCreate(ev));
  return FTX_OK;
}

// Launch wrapper: optional event pair on the launch stream around one step.
template <typename F>
ftx_status run_step(ftx_encoder* e, int step, hipStream_t s, F&& launch) {
  ftx_encoder::Mark m{nullptr, nullptr, step};
  if (e->timing) {
    ftx_status st = take_event(e, &m.start);
    if (st != FTX_OK) return st;
    if ((st = take_event(e, &m.stop)) != FTX_OK) return st;
    FTX_HIP(hipEventRecord(m.start, s));
  }
  hipError_t err = launch();
  if (err != hipSuccess) return hip_fail(err, "kernel launch");
  if (e->timing) {
    FTX_HIP(hipEventRecord(m.stop, s));
    e->marks.push_back(m);
  }
  return FTX_OK;
}

}  // namespace

namespace {

void drop_graph(ftx_encoder* e) {
  if (e->graph_exec) hipGraphExecDestroy(e->graph_exec);
  if (e->graph) hipGraphDestroy(e->graph);
  e->graph_exec = nullptr;
  e->graph = nullptr;
  e->g_in = e->g_out = nullptr;
  e->g_lens = nullptr;
}

// The projection with the attention in its epilogue replaces the projection + attention
// pair when the shape fits and, in the default mode, when there are at least 256 tokens and
// 64 tiles of 256 rows.  Below that the tiles are mostly padding rows or the long epilogue
// runs on few CUs, while the separate kernels spread the same work.  Measured, fused against
// separate (128-row tiles below 256 tiles of 256 rows): BERT-base S32 B1 0.482 against 0.462
// ms, B8 0.510 against 0.466, B12 0.529 against 0.482, B16 0.691 against 0.670, B64 0.805
// against 0.867; S64 B4 0.522 against 0.485, S64 B64 1.253 against 1.508; BERT-large S128 B2
// 1.431 against 1.280; the 4 x 32 model B64 0.294 against 0.296, B512 0.464 against 0.514.
// (Small batches once took the fused kernel whenever the separate Q/K/V projection split
// K; with that split capped it no longer pays.)
bool use_fused_attention(const ftx_encoder* e) {
  if (!e->fused || !e->attn_fits || e->fused_attention == 0) return false;
  if (e->fused_attention == 2) return true;
  return fused_attention_pays(e->T, e->H, e->dev.cus);
}

// The workspace of ftx_forward_static_workspace: FTX_STATIC_SCRATCH_BYTES of device memory
// per GPU, part of the library's code object (each device that runs the library holds its
// own copy until the process ends).  Host code must not pass `scratch` itself to a kernel --
// on the host the name stands for a host-side shadow, not the device array -- but the
// address static_scratch() obtains for the current device.
__device__ __align__(256) static char scratch[FTX_STATIC_SCRATCH_BYTES];

// Device address of `scratch` on device `dev` (which must be current), looked up with
// hipGetSymbolAddress the first time per device and kept; null if the lookup fails.
void* static_scratch(int dev) {
  static std::mutex mu;
  static std::vector<void*> addr;  // per device id
  if (dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if ((size_t)dev < addr.size() && addr[dev]) return addr[dev];
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();
    return nullptr;
  }
  if ((size_t)dev >= addr.size()) addr.resize(dev + 1, nullptr);
  addr[dev] = p;
  return p;
}

// Lay the workspace of `e` out from `base` into `w` (base null: only measure); returns its
// size in bytes.  Every view starts on a 256-byte boundary.
size_t layout_workspace(const ftx_encoder* e, char* base, Workspace* w) {
  auto pad = [](size_t bytes) { return (bytes + 255) / 256 * 256; };
  const size_t H = e->H, F = e->F, T = e->T, es = e->es;
  const size_t TH = pad(T * H * es);
  // bf16 keeps what enters a LayerNorm un-normalised in fp32: the residual Y1 and the two
  // projection outputs added to a residual (C Wo, G W2).  Half an ulp of bf16 at |v| in
  // [2, 4) is 7.8e-3, and the LayerNorms pass such errors to the output with gain ~gamma.
  const bool f32res = e->dt == FTX_BF16;
  const bool padded = e->Sv != e->S;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += pad(bytes);
    return p;
  };
  Workspace v;
  v.q = take(TH);
  v.k = take(TH);
  v.vt = take(TH);
  v.ctx = take(TH);
  v.abuf = take(f32res ? T * H * 4 : TH);
  v.y1 = take(TH);
  v.u = take(T * F * es);
  if (f32res) v.y1f = (float*)take(T * H * 4);
  if (e->fold_fits) v.st1 = (float*)take(T * e->ln1_ntn * 2 * sizeof(float));
  if (padded) {
    // the rows past Sv of each sequence are zero in the input copy and finite in the state;
    // neither reaches a row below Sv
    v.xpad = take(TH);
    v.spad = take(TH);
  }
  if (e->splitk_need) {
    v.splitk = (float*)take(e->splitk_need * sizeof(float));
    v.splitk_elems = e->splitk_need;
  }
  if (w) *w = v;
  return off;
}

// Enqueue the L-layer forward on `s` with the intermediate tensors of `ws` (arguments already
// validated).  clear_pad: zero the padded input copy first (a workspace shared with other
// forwards may hold anything there; the handle's own is zeroed once at create).
ftx_status enqueue_forward(ftx_encoder* e, const Workspace& ws, const void* input,
                           const int32_t* seq_lens, void* output, hipStream_t s,
                           bool clear_pad = false) {
  const ftx_dtype dt = e->dt;
  const int B = e->B, S = e->S, nh = e->nh, d = e->d, H = e->H, F = e->F, T = e->T;
  // The stack's state lives in `output`, or -- when the caller's length Sv is not a multiple
  // of 32 -- in the padded buffers: the input is copied to rows 0..Sv-1 of each sequence's
  // S rows, the layers run at S, and rows 0..Sv-1 are copied back at the end.
  const void* x0 = input;
  void* state = output;
  if (ws.xpad) {
    const size_t row = (size_t)H * e->es;
    if (clear_pad) FTX_HIP(launch_zero(ws.xpad, (size_t)B * S * row, s));
    FTX_HIP(hipMemcpy2DAsync(ws.xpad, S * row, input, e->Sv * row, e->Sv * row, B,
                             hipMemcpyDeviceToDevice, s));
    x0 = ws.xpad;
    state = ws.spad;
  }
  for (int l = 0; l < e->L; ++l) {
    const LayerW& w = e->layers[l];
    const void* x = (l == 0) ? x0 : state;
    ftx_status st;
    if (use_fused_attention(e)) {
      st = run_step(e, FTX_STEP_QKV_ATTENTION, s, [&] {
        return launch_qkv_attention(dt, B, S, nh, d, x, w.w_qkvh_t, w.b_qkvh, seq_lens, e->Sv,
                                    ws.ctx, s);
      });
    } else if (e->fused) {
      st = run_step(e, FTX_STEP_QKV_GEMM, s, [&] {
        return launch_qkv_projection(dt, B, S, nh, d, x, w.w_qkv_t, w.b_qkv, ws.q, ws.k, ws.vt, s,
                                     ws.splitk, ws.splitk_elems);
      });
    } else {
      st = run_step(e, FTX_STEP_QKV_GEMM, s, [&] {
        return launch_linear(dt, T, 3 * H, H, x, w.w_qkv_t, nullptr, false, ws.u, s, false,
                             ws.splitk, ws.splitk_elems);
      });
      if (st != FTX_OK) return st;
      st = run_step(e, FTX_STEP_BIAS_QKV_SPLIT, s, [&] {
        return launch_bias_qkv_split(dt, B, S, nh, d, ws.u, w.b_qkv, ws.q, ws.k, ws.vt, s);
      });
    }
    if (st != FTX_OK) return st;
    // Hidden size 128 with at least 128 row tiles: one 64 x 128 projection tile holds whole
    // rows, and the projection runs the bias + residual + LayerNorm in its epilogue (the
    // 4 x 32 model at batch 512: 0.445 -> 0.418 ms; with fewer tiles the unsplit K chain on
    // few CUs loses -- batch 64 0.302 -> 0.338 ms).  Otherwise a projection that splits K
    // (small batches) leaves its fp32 partials to the LayerNorm that follows it, which sums
    // them itself: one launch instead of reduction + LayerNorm.  At S = 32 such a split runs
    // by head inside the attention kernel instead (its K range is the merged-heads dimension):
    // one launch for the attention and the projection.
    const bool row_ln = H == 128 && (T + 63) / 64 >= 128;
    // The first LayerNorm folded into the first FFN projection (16-bit data at batches whose
    // projections do not split K): LN1(z) W1 + b1 = r (z (gamma o W1)) + s colsum(gamma o W1)
    // + (b1 + beta W1) with the row's r = 1/sigma and s = -mean/sigma.  The attention-output
    // projection stores Z1 = x + C Wo + bo (bf16: also in fp32) and per-tile (mean, M2) of
    // each row; the FFN-in projection merges the pairs and applies r, s in its epilogue; the
    // second LayerNorm rebuilds its residual Y1 = LN1(Z1) from Z1 (bf16: the fp32 copy, with
    // the FFN-out branch in fp32 as in the unfolded path) and the same pairs.  Four launches
    // after the attention instead of five.
    if (e->fold && e->fold_fits && e->fused && !row_ln) {
      if (!use_fused_attention(e)) {
        st = run_step(e, FTX_STEP_ATTENTION, s, [&] {
          return launch_attention(dt, B, S, S, nh, d, ws.q, ws.k, ws.vt, seq_lens, ws.ctx, s, e->Sv);
        });
        if (st != FTX_OK) return st;
      }
      st = run_step(e, FTX_STEP_ATTN_OUT_GEMM, s, [&] {
        return launch_linear_residual_stats(dt, T, H, H, ws.ctx, w.w_o_t, w.b_o, x, ws.y1,
                                            ws.y1f, ws.st1, e->ln1_ntn, s);
      });
      if (st != FTX_OK) return st;
      // FFN-in, FFN-out and the second LayerNorm in row chunks (ffn_rows rows; all rows but at
      // the largest batches), so that a chunk's F-wide intermediate stays in the last-level
      // cache between the two projections
      const bool f32res = ws.y1f != nullptr;  // bf16: Z1 and the FFN-out branch in fp32
      const size_t eh = f32res ? sizeof(float) : e->es;
      for (int r0 = 0; r0 < T; r0 += e->ffn_rows) {
        const int m = std::min(e->ffn_rows, T - r0);
        const size_t ro = (size_t)r0 * H;
        const float* st1 = ws.st1 + (size_t)r0 * e->ln1_ntn * 2;
        st = run_step(e, FTX_STEP_FFN1_GEMM, s, [&] {
          return launch_linear_norm_in(dt, m, F, H, (const char*)ws.y1 + ro * e->es, w.w1g_t, w.b1f,
                                       w.c1, st1, e->ln1_ntn, e->ln1_bn, true, ws.u, s);
        });
        if (st != FTX_OK) return st;
        if (r0 == 0 && (e->prefetch == 2 || (e->prefetch == 1 && e->w2_prefetch_fits))) {
          st = run_step(e, FTX_STEP_PREFETCH, s, [&] {
            return launch_prefetch(w.w2_t, (size_t)H * F * e->es, s);
          });
          if (st != FTX_OK) return st;
        }
        st = run_step(e, FTX_STEP_FFN2_GEMM, s, [&] {
          return launch_linear(dt, m, H, F, ws.u, w.w2_t, nullptr, false, (char*)ws.abuf + ro * eh,
                               s, f32res, ws.splitk, ws.splitk_elems);
        });
        if (st != FTX_OK) return st;
        st = run_step(e, FTX_STEP_LN2, s, [&] {
          const void* zx = f32res ? (const void*)((const char*)ws.y1f + ro * eh) : (const char*)ws.y1 + ro * e->es;
          return launch_bias_residual_layernorm_xnorm(dt, m, H, zx, f32res, st1, e->ln1_ntn, e->ln1_bn,
                                                      w.ln1_g, w.ln1_b, (const char*)ws.abuf + ro * eh,
                                                      f32res, w.b2, w.ln2_g, w.ln2_b,
                                                      (char*)state + ro * e->es, s);
        });
        if (st != FTX_OK) return st;
      }
      continue;
    }
    const int o_splits = linear_splits(dt, T, H, H, ws.splitk_elems, true);
    const bool attn_out = e->attn_out && !use_fused_attention(e) && e->fused && !row_ln &&
                          o_splits > 1 && (size_t)nh * T * H <= ws.splitk_elems;
    if (attn_out) {
      st = run_step(e, FTX_STEP_ATTENTION, s, [&] {
        return launch_attention_out_partials(dt, B, nh, d, ws.q, ws.k, ws.vt, seq_lens, e->Sv,
                                             w.w_o_t, ws.splitk, s);
      });
      if (st != FTX_OK) return st;
      st = run_step(e, FTX_STEP_LN1, s, [&] {
        return launch_splitk_bias_residual_layernorm(dt, T, H, x, false, ws.splitk, nh,
                                                     ws.y1f != nullptr, w.b_o, w.ln1_g, w.ln1_b,
                                                     ws.y1, ws.y1f, s);
      });
    } else {
      if (!use_fused_attention(e)) {
        st = run_step(e, FTX_STEP_ATTENTION, s, [&] {
          return launch_attention(dt, B, S, S, nh, d, ws.q, ws.k, ws.vt, seq_lens, ws.ctx, s, e->Sv);
        });
        if (st != FTX_OK) return st;
      }
      if (row_ln) {
        st = run_step(e, FTX_STEP_ATTN_OUT_GEMM, s, [&] {
          return launch_linear_layernorm(dt, T, H, H, ws.ctx, w.w_o_t, x, false, ws.y1f != nullptr,
                                         w.b_o, w.ln1_g, w.ln1_b, ws.y1, ws.y1f, s);
        });
      } else if (o_splits > 1) {
        st = run_step(e, FTX_STEP_ATTN_OUT_GEMM, s, [&] {
          return launch_linear_partials(dt, T, H, H, ws.ctx, w.w_o_t, ws.splitk, ws.splitk_elems, s);
        });
        if (st != FTX_OK) return st;
        st = run_step(e, FTX_STEP_LN1, s, [&] {
          return launch_splitk_bias_residual_layernorm(dt, T, H, x, false, ws.splitk, o_splits,
                                                       ws.y1f != nullptr, w.b_o, w.ln1_g, w.ln1_b,
                                                       ws.y1, ws.y1f, s);
        });
      } else {
        st = run_step(e, FTX_STEP_ATTN_OUT_GEMM, s, [&] {
          return launch_linear(dt, T, H, H, ws.ctx, w.w_o_t, nullptr, false, ws.abuf, s,
                               ws.y1f != nullptr, ws.splitk, ws.splitk_elems);
        });
        if (st != FTX_OK) return st;
        st = run_step(e, FTX_STEP_LN1, s, [&] {
          if (ws.y1f)
            return launch_bias_residual_layernorm_f32res(dt, T, H, x, false, (const float*)ws.abuf,
                                                         w.b_o, w.ln1_g, w.ln1_b, ws.y1, ws.y1f, s);
          return launch_bias_residual_layernorm(dt, T, H, x, ws.abuf, w.b_o, w.ln1_g, w.ln1_b, ws.y1, s);
        });
      }
    }
    if (st != FTX_OK) return st;
    if (e->fused) {
      st = run_step(e, FTX_STEP_FFN1_GEMM, s, [&] {
        return launch_linear(dt, T, F, H, ws.y1, w.w1_t, w.b1, true, ws.u, s, false, ws.splitk,
                             ws.splitk_elems);
      });
    } else {
      st = run_step(e, FTX_STEP_FFN1_GEMM, s, [&] {
        return launch_linear(dt, T, F, H, ws.y1, w.w1_t, nullptr, false, ws.u, s, false, ws.splitk,
                             ws.splitk_elems);
      });
      if (st != FTX_OK) return st;
      st = run_step(e, FTX_STEP_BIAS_GELU, s, [&] {
        return launch_bias_gelu(dt, T, F, ws.u, w.b1, ws.u, s);
      });
    }
    if (st != FTX_OK) return st;
    const int f_splits = linear_splits(dt, T, H, F, ws.splitk_elems, true);
    if (row_ln) {
      st = run_step(e, FTX_STEP_FFN2_GEMM, s, [&] {
        const bool f32res = ws.y1f != nullptr;
        return launch_linear_layernorm(dt, T, H, F, ws.u, w.w2_t,
                                       f32res ? (const void*)ws.y1f : ws.y1, f32res, f32res,
                                       w.b2, w.ln2_g, w.ln2_b, state, nullptr, s);
      });
    } else if (f_splits > 1) {
      st = run_step(e, FTX_STEP_FFN2_GEMM, s, [&] {
        return launch_linear_partials(dt, T, H, F, ws.u, w.w2_t, ws.splitk, ws.splitk_elems, s);
      });
      if (st != FTX_OK) return st;
      st = run_step(e, FTX_STEP_LN2, s, [&] {
        const bool f32res = ws.y1f != nullptr;
        return launch_splitk_bias_residual_layernorm(dt, T, H, f32res ? (const void*)ws.y1f : ws.y1,
                                                     f32res, ws.splitk, f_splits, f32res, w.b2,
                                                     w.ln2_g, w.ln2_b, state, nullptr, s);
      });
    } else {
      st = run_step(e, FTX_STEP_FFN2_GEMM, s, [&] {
        return launch_linear(dt, T, H, F, ws.u, w.w2_t, nullptr, false, ws.abuf, s,
                             ws.y1f != nullptr, ws.splitk, ws.splitk_elems);
      });
      if (st != FTX_OK) return st;
      st = run_step(e, FTX_STEP_LN2, s, [&] {
        if (ws.y1f)
          return launch_bias_residual_layernorm_f32res(dt, T, H, ws.y1f, true, (const float*)ws.abuf, w.b2,
                                                       w.ln2_g, w.ln2_b, state, nullptr, s);
        return launch_bias_residual_layernorm(dt, T, H, ws.y1, ws.abuf, w.b2, w.ln2_g, w.ln2_b, state, s);
      });
    }
    if (st != FTX_OK) return st;
  }
  if (ws.xpad) {
    const size_t row = (size_t)H * e->es;
    FTX_HIP(hipMemcpy2DAsync(output, e->Sv * row, state, S * row, e->Sv * row, B,
                             hipMemcpyDeviceToDevice, s));
  }
  return FTX_OK;
}

}  // namespace

extern "C" {

const char* ftx_status_string(ftx_status s) {
  switch (s) {
    case FTX_OK: return "ok";
    case FTX_ERR_INVALID_ARG: return "invalid argument";
    case FTX_ERR_UNSUPPORTED: return "unsupported";
    case FTX_ERR_OUT_OF_MEMORY: return "out of device memory";
    case FTX_ERR_DEVICE: return "device error";
    case FTX_ERR_NOT_READY: return "weights not set";
  }
  return "unknown status";
}

const char* ftx_last_error(void) { return last_error_slot().c_str(); }

ftx_status ftx_encoder_create(int batch_size, int seq_len, int head_num, int size_per_head,
                              int num_layers, ftx_dtype dtype, ftx_encoder** out) {
  last_error_slot().clear();
  if (!out) return fail(FTX_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  if (num_layers < 1) return fail(FTX_ERR_INVALID_ARG, "num_layers must be >= 1");
  ftx_status st = check_shape(batch_size, seq_len, head_num, size_per_head, true);
  if (st != FTX_OK) return st;

  int dev = 0;
  FTX_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  FTX_HIP(hipGetDeviceProperties(&prop, dev));
  if (std::string(prop.gcnArchName).rfind("gfx950", 0) != 0)
    return fail(FTX_ERR_UNSUPPORTED, std::string("built for gfx950, device is ") + prop.gcnArchName);

  ftx_encoder* e = new (std::nothrow) ftx_encoder();
  if (!e) return fail(FTX_ERR_OUT_OF_MEMORY, "host allocation");
  e->B = batch_size;
  e->Sv = seq_len;
  e->S = (seq_len + 31) / 32 * 32;
  e->nh = head_num;
  e->d = size_per_head;
  e->L = num_layers;
  e->H = head_num * size_per_head;
  e->F = 4 * e->H;
  e->T = batch_size * e->S;
  e->dt = dtype;
  e->es = dtype_size(dtype);
  e->device = dev;
  e->dev = device_info();

  e->attn_fits = qkv_attention_fits(dtype, e->S, head_num, size_per_head);

  const size_t H = e->H, F = e->F, T = e->T, es = e->es;
  // split-K workspace: the largest any of the four projections plans for, and the per-head
  // partials of the attention-output projection where the attention produces them (S = 32,
  // the projection splits, and the partials stay within 4 MiB: BERT-base up to 3 sequences;
  // at batch 8, 9 MiB of partials made the forward slower than the separate projection,
  // 0.474 against 0.467 ms)
  e->splitk_need = std::max(std::max(gemm_splitk_workspace(dtype, e->T, 3 * e->H, e->H),
                                     gemm_splitk_workspace(dtype, e->T, e->H, e->H)),
                            std::max(gemm_splitk_workspace(dtype, e->T, e->F, e->H),
                                     gemm_splitk_workspace(dtype, e->T, e->H, e->F)));
  {
    const size_t per_head = (size_t)head_num * e->T * e->H;
    e->attn_out = attention_out_partials_fit(dtype, e->S, head_num, size_per_head) &&
                  linear_splits(dtype, e->T, e->H, e->H, (size_t)1 << 40, true) > 1 &&
                  per_head * sizeof(float) <= (4u << 20);
    if (e->attn_out) e->splitk_need = std::max(e->splitk_need, per_head);
  }
  {
    // the LayerNorm fold: 16-bit data, the hidden sizes the rebuilding LayerNorm tiles
    // exactly, and unsplit projections on multi-wave tiles for the attention output, FFN-in
    // and FFN-out
    int tm, tn, sp, tm1, tn1, sp1;
    plan_linear(dtype, e->T, e->H, e->H, e->dev.cus, false, &tm, &tn, &sp);
    plan_linear(dtype, e->T, e->F, e->H, e->dev.cus, false, &tm1, &tn1, &sp1);
    e->fold_fits = (dtype == FTX_FP16 || dtype == FTX_BF16) && (e->H == 768 || e->H == 1024) && !e->attn_out &&
                   sp == 1 && tm > 32 && sp1 == 1 && tm1 > 32 &&
                   linear_splits(dtype, e->T, e->H, e->H, (size_t)1 << 40, true) == 1 &&
                   linear_splits(dtype, e->T, e->H, e->F, (size_t)1 << 40, true) == 1;
    if (e->fold_fits) {
      e->ln1_bn = tn;
      e->ln1_ntn = (e->H + tn - 1) / tn;
      // FFN chunks: the F-wide intermediate of a chunk within kFfnChunkBytes, chunks of whole
      // 256-row tiles, each still planned unsplit
      e->ffn_rows = e->T;
      const size_t u_bytes = (size_t)e->T * e->F * e->es;
      if (u_bytes > kFfnChunkBytes) {
        const int n = (int)((u_bytes + kFfnChunkBytes - 1) / kFfnChunkBytes);
        const int rows = ((e->T + n - 1) / n + 255) / 256 * 256;
        int tm2, tn2, sp2;
        plan_linear(dtype, rows, e->F, e->H, e->dev.cus, false, &tm2, &tn2, &sp2);
        if (sp2 == 1 && tm2 > 32 && linear_splits(dtype, rows, e->H, e->F, (size_t)1 << 40, true) == 1)
          e->ffn_rows = rows;
      }
      // The second FFN projection reads its weights cold: every layer's weights and
      // activations pass through the last-level cache between two reads of a layer's W2.  On
      // 128-row tiles with at least 1.5 tiles per CU (two blocks on most CUs, all resident at
      // once, each with one slab in flight) the cold W2 slows it most: BERT-base 8192 rows 59 -> 44 us
      // with W2 read just before it by a separate 5 us kernel; whole forwards (same box) S32
      // B256 2.19 -> 2.05 ms, S128 B64 2.24 -> 2.10, BERT-large S128 B64 5.99 -> 5.79, S32
      // B192 1.82 -> 1.79.  With fewer tiles (4096 rows) or 256-row tiles it loses by about
      // the prefetch's own time.
      {
        int tm3, tn3, sp3;
        plan_linear(dtype, e->ffn_rows, e->H, e->F, e->dev.cus, true, &tm3, &tn3, &sp3);
        const int64_t tiles3 = (int64_t)((e->ffn_rows + tm3 - 1) / tm3) * ((e->H + tn3 - 1) / tn3);
        e->w2_prefetch_fits = tm3 == 128 && (tn3 == 128 || tn3 == 96) && sp3 == 1 &&
                              2 * tiles3 >= 3 * (int64_t)e->dev.cus;
      }
    }
  }
  // weights: per layer 3H*H + 3H + H*H + H + 2H + F*H + F + H*F + H + 2H elements (plus a
  // second 3H*H + 3H in per-head order for the fused attention, and for the LayerNorm fold
  // F*H more plus 2F fp32), each tensor padded to 256 bytes
  auto pad = [](size_t bytes) { return (bytes + 255) / 256 * 256; };
  const size_t per_layer = pad(3 * H * H * es) + pad(3 * H * es) + pad(H * H * es) + 5 * pad(H * es) +
                           pad(F * H * es) + pad(F * es) + pad(H * F * es) + pad(H * es) +
                           (e->attn_fits ? pad(3 * H * H * es) + pad(3 * H * es) : 0) +
                           (e->fold_fits ? pad(F * H * es) + 2 * pad(F * 4) : 0);
  hipError_t err = hipMalloc(&e->weights, per_layer * e->L);
  if (err != hipSuccess) {
    delete e;
    return hip_fail(err, "hipMalloc(weights)");
  }
  e->ws_bytes = layout_workspace(e, nullptr, nullptr);
  err = hipMalloc(&e->ws_mem, e->ws_bytes);
  if (err != hipSuccess) {
    hipFree(e->weights);
    delete e;
    return hip_fail(err, "hipMalloc(workspace)");
  }
  layout_workspace(e, (char*)e->ws_mem, &e->w);
  char* w = (char*)e->weights;
  e->layers.resize(e->L);
  for (int l = 0; l < e->L; ++l) {
    LayerW& lw = e->layers[l];
    auto take = [&](size_t bytes) { void* p = w; w += pad(bytes); return p; };
    lw.w_qkv_t = take(3 * H * H * es);
    lw.b_qkv = take(3 * H * es);
    lw.w_o_t = take(H * H * es);
    lw.b_o = take(H * es);
    lw.ln1_g = take(H * es);
    lw.ln1_b = take(H * es);
    lw.w1_t = take(F * H * es);
    lw.b1 = take(F * es);
    lw.w2_t = take(H * F * es);
    lw.b2 = take(H * es);
    lw.ln2_g = take(H * es);
    lw.ln2_b = take(H * es);
    lw.w_qkvh_t = e->attn_fits ? take(3 * H * H * es) : nullptr;
    lw.b_qkvh = e->attn_fits ? take(3 * H * es) : nullptr;
    if (e->fold_fits) {
      lw.w1g_t = take(F * H * es);
      lw.c1 = (float*)take(F * 4);
      lw.b1f = (float*)take(F * 4);
    }
  }
  e->ready.assign(e->L, 0);
  if (e->w.xpad) {
    // the rows past Sv of each sequence stay zero in the handle's input copy (nothing else
    // writes them)
    const size_t TH = (size_t)T * H * es;
    err = hipMemset(e->w.xpad, 0, TH);
    if (err == hipSuccess) err = hipMemset(e->w.spad, 0, TH);
    if (err == hipSuccess) err = hipDeviceSynchronize();
    if (err != hipSuccess) {
      hipFree(e->ws_mem);
      hipFree(e->weights);
      delete e;
      return hip_fail(err, "hipMemset(padding)");
    }
  }
  // the static scratch of ftx_forward_static_workspace, resolved once per device here (the
  // regular forward does not need it: a failure is reported by that entry point)
  (void)static_scratch(dev);
  *out = e;
  return FTX_OK;
}

ftx_status ftx_set_weights(ftx_encoder* e, int layer, const ftx_layer_weights* w, void* stream) {
  last_error_slot().clear();
  if (!e) return fail(FTX_ERR_INVALID_ARG, "encoder is NULL");
  if (!w) return fail(FTX_ERR_INVALID_ARG, "weights struct is NULL");
  if (layer < 0 || layer >= e->L) return fail(FTX_ERR_INVALID_ARG, "layer out of range");
  const void* ptrs[] = {w->w_q, w->b_q, w->w_k, w->b_k, w->w_v, w->b_v, w->w_o, w->b_o,
                        w->ln1_gamma, w->ln1_beta, w->w_ffn1, w->b_ffn1, w->w_ffn2, w->b_ffn2,
                        w->ln2_gamma, w->ln2_beta};
  for (const void* p : ptrs)
    if (!p) return fail(FTX_ERR_INVALID_ARG, "a weight pointer is NULL");
  for (const void* p : ptrs)
    if (!is_device_ptr(p)) return fail(FTX_ERR_INVALID_ARG, "a weight pointer is not device memory");
  hipStream_t s = (hipStream_t)stream;
  FTX_HIP(hipSetDevice(e->device));
  const size_t H = e->H, F = e->F, es = e->es;
  LayerW& lw = e->layers[layer];
  char* qkv = (char*)lw.w_qkv_t;
  FTX_HIP(launch_transpose(e->dt, e->H, e->H, w->w_q, qkv, s));
  FTX_HIP(launch_transpose(e->dt, e->H, e->H, w->w_k, qkv + H * H * es, s));
  FTX_HIP(launch_transpose(e->dt, e->H, e->H, w->w_v, qkv + 2 * H * H * es, s));
  FTX_HIP(launch_transpose(e->dt, e->H, e->H, w->w_o, lw.w_o_t, s));
  FTX_HIP(launch_transpose(e->dt, e->H, e->F, w->w_ffn1, lw.w1_t, s));
  FTX_HIP(launch_transpose(e->dt, e->F, e->H, w->w_ffn2, lw.w2_t, s));
  char* bqkv = (char*)lw.b_qkv;
  FTX_HIP(hipMemcpyAsync(bqkv, w->b_q, H * es, hipMemcpyDeviceToDevice, s));
  FTX_HIP(hipMemcpyAsync(bqkv + H * es, w->b_k, H * es, hipMemcpyDeviceToDevice, s));
  FTX_HIP(hipMemcpyAsync(bqkv + 2 * H * es, w->b_v, H * es, hipMemcpyDeviceToDevice, s));
  FTX_HIP(hipMemcpyAsync(lw.b_o, w->b_o, H * es, hipMemcpyDeviceToDevice, s));
  FTX_HIP(hipMemcpyAsync(lw.ln1_g, w->ln1_gamma, H * es, hipMemcpyDeviceToDevice, s));
  FTX_HIP(hipMemcpyAsync(lw.ln1_b, w->ln1_beta, H * es, hipMemcpyDeviceToDevice, s));
  FTX_HIP(hipMemcpyAsync(lw.b1, w->b_ffn1, F * es, hipMemcpyDeviceToDevice, s));
  FTX_HIP(hipMemcpyAsync(lw.b2, w->b_ffn2, H * es, hipMemcpyDeviceToDevice, s));
  FTX_HIP(hipMemcpyAsync(lw.ln2_g, w->ln2_gamma, H * es, hipMemcpyDeviceToDevice, s));
  FTX_HIP(hipMemcpyAsync(lw.ln2_b, w->ln2_beta, H * es, hipMemcpyDeviceToDevice, s));
  if (lw.w_qkvh_t) {
    // rows of head h of Q (K, V) go to rows 3 d h .. (+d, +2d)
    const size_t d = e->d;
    for (int part = 0; part < 3; ++part) {
      FTX_HIP(hipMemcpy2DAsync((char*)lw.w_qkvh_t + part * d * H * es, 3 * d * H * es,
                               qkv + part * H * H * es, d * H * es, d * H * es, e->nh,
                               hipMemcpyDeviceToDevice, s));
      FTX_HIP(hipMemcpy2DAsync((char*)lw.b_qkvh + part * d * es, 3 * d * es, bqkv + part * H * es,
                               d * es, d * es, e->nh, hipMemcpyDeviceToDevice, s));
    }
  }
  if (lw.w1g_t)
    FTX_HIP(launch_fold_layernorm_weights(e->dt, e->F, e->H, lw.w1_t, lw.ln1_g, lw.ln1_b, lw.b1,
                                          lw.w1g_t, lw.c1, lw.b1f, s));
  FTX_HIP(hipStreamSynchronize(s));
  e->ready[layer] = 1;
  return FTX_OK;
}

// Argument checks of the two forward entry points.
static ftx_status check_forward(const ftx_encoder* e, const void* input, const int32_t* seq_lens,
                                const void* output) {
  if (!e) return fail(FTX_ERR_INVALID_ARG, "encoder is NULL");
  if (!input || !output) return fail(FTX_ERR_INVALID_ARG, "input or output is NULL");
  if (!aligned16(input) || !aligned16(output))
    return fail(FTX_ERR_INVALID_ARG, "input and output must be 16-byte aligned");
  const size_t bytes = (size_t)e->B * e->Sv * e->H * e->es;  // caller's [B][Sv][H]
  if (overlap(input, bytes, output, bytes)) return fail(FTX_ERR_INVALID_ARG, "output overlaps input");
  for (int l = 0; l < e->L; ++l)
    if (!e->ready[l]) return fail(FTX_ERR_NOT_READY, "layer " + std::to_string(l) + " has no weights");
  if (!all_device({input, output, seq_lens}))
    return fail(FTX_ERR_INVALID_ARG, "input, output and seq_lens must be device memory");
  return FTX_OK;
}

ftx_status ftx_forward(ftx_encoder* e, const void* input, const int32_t* seq_lens, void* output,
                       void* stream) {
  last_error_slot().clear();
  ftx_status st0 = check_forward(e, input, seq_lens, output);
  if (st0 != FTX_OK) return st0;
  hipStream_t s = (hipStream_t)stream;
  FTX_HIP(hipSetDevice(e->device));
  if (!e->graph_mode || e->timing) return enqueue_forward(e, e->w, input, seq_lens, output, s);

  // graph mode: replay the captured forward if it was made for these buffers, else capture
  // one on the handle's own stream (the caller's may be the default stream, which cannot be
  // captured) and replay it on the caller's stream
  if (!(e->graph_exec && e->g_in == input && e->g_lens == seq_lens && e->g_out == output)) {
    drop_graph(e);
    if (!e->cap_stream) FTX_HIP(hipStreamCreateWithFlags(&e->cap_stream, hipStreamNonBlocking));
    FTX_HIP(hipStreamBeginCapture(e->cap_stream, hipStreamCaptureModeThreadLocal));
    ftx_status st = enqueue_forward(e, e->w, input, seq_lens, output, e->cap_stream);
    hipGraph_t g = nullptr;
    hipError_t err = hipStreamEndCapture(e->cap_stream, &g);
    if (st != FTX_OK) {
      if (g) hipGraphDestroy(g);
      return st;
    }
    if (err != hipSuccess) return hip_fail(err, "hipStreamEndCapture");
    e->graph = g;
    err = hipGraphInstantiate(&e->graph_exec, g, nullptr, nullptr, 0);
    if (err != hipSuccess) {
      drop_graph(e);
      return hip_fail(err, "hipGraphInstantiate");
    }
    e->g_in = input;
    e->g_lens = seq_lens;
    e->g_out = output;
  }
  FTX_HIP(hipGraphLaunch(e->graph_exec, s));
  return FTX_OK;
}

ftx_status ftx_forward_static_workspace(ftx_encoder* e, const void* input,
                                        const int32_t* seq_lens, void* output, void* stream) {
  last_error_slot().clear();
  ftx_status st = check_forward(e, input, seq_lens, output);
  if (st != FTX_OK) return st;
  if (e->ws_bytes > (size_t)FTX_STATIC_SCRATCH_BYTES)
    return fail(FTX_ERR_UNSUPPORTED,
                "this forward needs " + std::to_string(e->ws_bytes) +
                    " bytes of workspace; the static scratch holds " +
                    std::to_string((size_t)FTX_STATIC_SCRATCH_BYTES));
  FTX_HIP(hipSetDevice(e->device));
  char* base = (char*)static_scratch(e->device);
  if (!base) return fail(FTX_ERR_DEVICE, "hipGetSymbolAddress of the static scratch failed");
  Workspace w;
  layout_workspace(e, base, &w);
  return enqueue_forward(e, w, input, seq_lens, output, (hipStream_t)stream, true);
}

ftx_status ftx_destroy(ftx_encoder* e) {
  last_error_slot().clear();
  if (!e) return FTX_OK;
  hipSetDevice(e->device);
  hipDeviceSynchronize();
  for (auto& m : e->marks) {
    hipEventDestroy(m.start);
    hipEventDestroy(m.stop);
  }
  for (auto ev : e->pool) hipEventDestroy(ev);
  drop_graph(e);
  if (e->cap_stream) hipStreamDestroy(e->cap_stream);
  hipFree(e->weights);
  hipFree(e->ws_mem);
  delete e;
  return FTX_OK;
}

ftx_status ftx_set_option(ftx_encoder* e, ftx_option option, int value) {
  last_error_slot().clear();
  if (!e) return fail(FTX_ERR_INVALID_ARG, "encoder is NULL");
  switch (option) {
    case FTX_OPT_FUSED_EPILOGUES:
      if (e->fused != (value ? 1 : 0)) drop_graph(e);  // the captured launch sequence changes
      e->fused = value ? 1 : 0;
      return FTX_OK;
    case FTX_OPT_KERNEL_TIMING: e->timing = value ? 1 : 0; return FTX_OK;
    case FTX_OPT_FUSED_ATTENTION:
      if (value < 0 || value > 2) return fail(FTX_ERR_INVALID_ARG, "fused attention mode is 0, 1 or 2");
      if (e->fused_attention != value) drop_graph(e);
      e->fused_attention = value;
      return FTX_OK;
    case FTX_OPT_GRAPH:
      e->graph_mode = value ? 1 : 0;
      if (!e->graph_mode) drop_graph(e);
      return FTX_OK;
    case FTX_OPT_FOLD_LAYERNORM:
      if (e->fold != (value ? 1 : 0)) drop_graph(e);
      e->fold = value ? 1 : 0;
      return FTX_OK;
    case FTX_OPT_PREFETCH_WEIGHTS:
      if (value < 0 || value > 2) return fail(FTX_ERR_INVALID_ARG, "weight prefetch mode is 0, 1 or 2");
      if (e->prefetch != value) drop_graph(e);
      e->prefetch = value;
      return FTX_OK;
  }
  return fail(FTX_ERR_INVALID_ARG, "unknown option");
}

ftx_status ftx_kernel_times(ftx_encoder* e, double* ms, int64_t* counts) {
  last_error_slot().clear();
  if (!e) return fail(FTX_ERR_INVALID_ARG, "encoder is NULL");
  double acc[FTX_NUM_STEPS] = {0};
  int64_t cnt[FTX_NUM_STEPS] = {0};
  for (auto& m : e->marks) {
    FTX_HIP(hipEventSynchronize(m.stop));
    float t = 0.f;
    FTX_HIP(hipEventElapsedTime(&t, m.start, m.stop));
    acc[m.step] += t;
    cnt[m.step] += 1;
    e->pool.push_back(m.start);
    e->pool.push_back(m.stop);
  }
  e->marks.clear();
  for (int i = 0; i < FTX_NUM_STEPS; ++i) {
    if (ms) ms[i] = acc[i];
    if (counts) counts[i] = cnt[i];
  }
  return FTX_OK;
}

// ------------------------------------------------------------------------ step entry points

ftx_status ftx_step_linear(ftx_dtype dtype, int M, int N, int K, const void* a, const void* w_t,
                           const void* bias, int gelu, void* c, void* stream) {
  last_error_slot().clear();
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  if (M < 1 || N < 8 || K < 8 || N % 8 || K % 8)
    return fail(FTX_ERR_INVALID_ARG, "need M >= 1 and N, K positive multiples of 8");
  if ((long long)M * N >= (1LL << 31) || (long long)M * K >= (1LL << 31) || (long long)N * K >= (1LL << 31))
    return fail(FTX_ERR_UNSUPPORTED, "operand above 2^31 elements");
  if (K > kMaxInnerDim) return fail(FTX_ERR_UNSUPPORTED, "K above 2^20");
  if (!a || !w_t || !c) return fail(FTX_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(a) || !aligned16(w_t) || !aligned16(c)) return fail(FTX_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t es = dtype_size(dtype);
  if (overlap(a, (size_t)M * K * es, c, (size_t)M * N * es) || overlap(w_t, (size_t)N * K * es, c, (size_t)M * N * es))
    return fail(FTX_ERR_INVALID_ARG, "output overlaps an input");
  if (!all_device({a, w_t, bias, c})) return fail(FTX_ERR_INVALID_ARG, "pointers must be device memory");
  hipError_t err = launch_linear(dtype, M, N, K, a, w_t, bias, gelu != 0, c, (hipStream_t)stream);
  return err == hipSuccess ? FTX_OK : hip_fail(err, "linear launch");
}

ftx_status ftx_step_qkv_projection(ftx_dtype dtype, int B, int S, int n, int d, const void* x,
                                   const void* w_qkv_t, const void* b_qkv, void* q, void* k,
                                   void* v_t, void* stream) {
  last_error_slot().clear();
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  ftx_status st = check_shape(B, S, n, d);
  if (st != FTX_OK) return st;
  if (!x || !w_qkv_t || !b_qkv || !q || !k || !v_t) return fail(FTX_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(x) || !aligned16(w_qkv_t) || !aligned16(q) || !aligned16(k) || !aligned16(v_t))
    return fail(FTX_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (!all_device({x, w_qkv_t, b_qkv, q, k, v_t})) return fail(FTX_ERR_INVALID_ARG, "pointers must be device memory");
  hipError_t err = launch_qkv_projection(dtype, B, S, n, d, x, w_qkv_t, b_qkv, q, k, v_t, (hipStream_t)stream);
  return err == hipSuccess ? FTX_OK : hip_fail(err, "qkv projection launch");
}

ftx_status ftx_step_bias_qkv_split(ftx_dtype dtype, int B, int S, int n, int d, const void* qkv,
                                   const void* b_qkv, void* q, void* k, void* v_t, void* stream) {
  last_error_slot().clear();
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  ftx_status st = check_shape(B, S, n, d);
  if (st != FTX_OK) return st;
  if (!qkv || !b_qkv || !q || !k || !v_t) return fail(FTX_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(qkv) || !aligned16(b_qkv) || !aligned16(q) || !aligned16(k) || !aligned16(v_t))
    return fail(FTX_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (!all_device({qkv, b_qkv, q, k, v_t})) return fail(FTX_ERR_INVALID_ARG, "pointers must be device memory");
  hipError_t err = launch_bias_qkv_split(dtype, B, S, n, d, qkv, b_qkv, q, k, v_t, (hipStream_t)stream);
  return err == hipSuccess ? FTX_OK : hip_fail(err, "bias qkv split launch");
}

ftx_status ftx_step_attention(ftx_dtype dtype, int B, int S, int n, int d, const void* q,
                              const void* k, const void* v_t, const int32_t* seq_lens, void* ctx,
                              void* stream) {
  last_error_slot().clear();
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  ftx_status st = check_shape(B, S, n, d);
  if (st != FTX_OK) return st;
  if (!q || !k || !v_t || !ctx) return fail(FTX_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v_t) || !aligned16(ctx))
    return fail(FTX_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (!all_device({q, k, v_t, seq_lens, ctx})) return fail(FTX_ERR_INVALID_ARG, "pointers must be device memory");
  hipError_t err = launch_attention(dtype, B, S, S, n, d, q, k, v_t, seq_lens, ctx, (hipStream_t)stream);
  return err == hipSuccess ? FTX_OK : hip_fail(err, "attention launch");
}

ftx_status ftx_step_qkv_attention(ftx_dtype dtype, int B, int S, int n, int d, const void* x,
                                  const void* w_qkv_t, const void* b_qkv, const int32_t* seq_lens,
                                  int causal, void* ctx, void* stream) {
  last_error_slot().clear();
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  ftx_status st = check_shape(B, S, n, d);
  if (st != FTX_OK) return st;
  if (!qkv_attention_fits(dtype, S, n, d))
    return fail(FTX_ERR_UNSUPPORTED,
                "fused projection + attention needs fp16/bf16, S in {32, 64, 128, 256}, d = 64 "
                "(or 32 with an even head count)");
  if (!x || !w_qkv_t || !b_qkv || !ctx) return fail(FTX_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(x) || !aligned16(w_qkv_t) || !aligned16(b_qkv) || !aligned16(ctx))
    return fail(FTX_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  // other tiles still read rows of x while a tile writes its context rows
  const size_t es = dtype_size(dtype), H = (size_t)n * d, rows = (size_t)B * S;
  if (overlap(x, rows * H * es, ctx, rows * H * es) || overlap(w_qkv_t, 3 * H * H * es, ctx, rows * H * es))
    return fail(FTX_ERR_INVALID_ARG, "ctx overlaps an input");
  if (!all_device({x, w_qkv_t, b_qkv, seq_lens, ctx}))
    return fail(FTX_ERR_INVALID_ARG, "pointers must be device memory");
  hipError_t err = launch_qkv_attention(dtype, B, S, n, d, x, w_qkv_t, b_qkv, seq_lens, S, ctx,
                                        (hipStream_t)stream, causal != 0);
  return err == hipSuccess ? FTX_OK : hip_fail(err, "qkv attention launch");
}

ftx_status ftx_step_masked_attention(ftx_dtype dtype, int B, int Sq, int Sk, int n, int d,
                                     const void* q, const void* k, const void* v_t,
                                     const int32_t* key_lens, int causal, void* ctx,
                                     void* stream) {
  last_error_slot().clear();
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  ftx_status st = check_shape(B, Sq, n, d);
  if (st == FTX_OK) st = check_shape(B, Sk, n, d);
  if (st != FTX_OK) return st;
  if (causal && Sq != Sk) return fail(FTX_ERR_INVALID_ARG, "causal attention needs Sq == Sk");
  if (!q || !k || !v_t || !ctx) return fail(FTX_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v_t) || !aligned16(ctx))
    return fail(FTX_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (!all_device({q, k, v_t, key_lens, ctx})) return fail(FTX_ERR_INVALID_ARG, "pointers must be device memory");
  hipError_t err = launch_attention(dtype, B, Sq, Sk, n, d, q, k, v_t, key_lens, ctx,
                                    (hipStream_t)stream, 0, causal != 0);
  return err == hipSuccess ? FTX_OK : hip_fail(err, "attention launch");
}

ftx_status ftx_step_bias_residual_layernorm(ftx_dtype dtype, int rows, int cols, const void* x,
                                            const void* a, const void* bias, const void* gamma,
                                            const void* beta, void* y, void* stream) {
  last_error_slot().clear();
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  if (rows < 1 || cols < 4 || cols % 4) return fail(FTX_ERR_INVALID_ARG, "need rows >= 1, cols a positive multiple of 4");
  if (cols > kMaxLayerNormCols) return fail(FTX_ERR_UNSUPPORTED, "cols above 4096");
  if ((long long)rows * cols >= (1LL << 31)) return fail(FTX_ERR_UNSUPPORTED, "tensor above 2^31 elements");
  if (!x || !a || !bias || !gamma || !beta || !y) return fail(FTX_ERR_INVALID_ARG, "NULL pointer");
  const size_t align = dtype_size(dtype) * 4;  // 4-element vector accesses
  for (const void* p : {x, a, bias, gamma, beta, (const void*)y})
    if ((uintptr_t)p % align) return fail(FTX_ERR_INVALID_ARG, "pointers must be aligned to 4 elements");
  if (!all_device({x, a, bias, gamma, beta, y})) return fail(FTX_ERR_INVALID_ARG, "pointers must be device memory");
  hipError_t err = launch_bias_residual_layernorm(dtype, rows, cols, x, a, bias, gamma, beta, y, (hipStream_t)stream);
  return err == hipSuccess ? FTX_OK : hip_fail(err, "layernorm launch");
}

ftx_status ftx_step_bias_gelu(ftx_dtype dtype, int rows, int cols, const void* u, const void* bias,
                              void* g, void* stream) {
  last_error_slot().clear();
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  if (rows < 1 || cols < 8 || cols % 8) return fail(FTX_ERR_INVALID_ARG, "need rows >= 1, cols a positive multiple of 8");
  if ((long long)rows * cols >= (1LL << 31)) return fail(FTX_ERR_UNSUPPORTED, "tensor above 2^31 elements");
  if (!u || !bias || !g) return fail(FTX_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(u) || !aligned16(bias) || !aligned16(g)) return fail(FTX_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (!all_device({u, bias, g})) return fail(FTX_ERR_INVALID_ARG, "pointers must be device memory");
  hipError_t err = launch_bias_gelu(dtype, rows, cols, u, bias, g, (hipStream_t)stream);
  return err == hipSuccess ? FTX_OK : hip_fail(err, "bias gelu launch");
}

ftx_status ftx_step_transpose(ftx_dtype dtype, int rows, int cols, const void* in, void* out,
                              void* stream) {
  last_error_slot().clear();
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  if (rows < 1 || cols < 1) return fail(FTX_ERR_INVALID_ARG, "need rows, cols >= 1");
  if ((long long)rows * cols >= (1LL << 31)) return fail(FTX_ERR_UNSUPPORTED, "tensor above 2^31 elements");
  if (!in || !out) return fail(FTX_ERR_INVALID_ARG, "NULL pointer");
  const size_t bytes = (size_t)rows * cols * dtype_size(dtype);
  if (overlap(in, bytes, out, bytes)) return fail(FTX_ERR_INVALID_ARG, "output overlaps input");
  if (!all_device({in, out})) return fail(FTX_ERR_INVALID_ARG, "pointers must be device memory");
  hipError_t err = launch_transpose(dtype, rows, cols, in, out, (hipStream_t)stream);
  return err == hipSuccess ? FTX_OK : hip_fail(err, "transpose launch");
}

ftx_status ftx_plan_linear(ftx_dtype dtype, int M, int N, int K, int cus, int sums_partials,
                           int* tile_m, int* tile_n, int* splits) {
  last_error_slot().clear();
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  if (M < 1 || N < 1 || K < 1 || cus < 1) return fail(FTX_ERR_INVALID_ARG, "M, N, K and cus must be >= 1");
  if (!tile_m || !tile_n || !splits) return fail(FTX_ERR_INVALID_ARG, "NULL pointer");
  plan_linear(dtype, M, N, K, cus, sums_partials != 0, tile_m, tile_n, splits);
  return FTX_OK;
}

}  // extern "C"
