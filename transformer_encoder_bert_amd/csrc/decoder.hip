// The C ABI of the ftx decoder: handle, weight repacking and the per-layer launch sequence.
// Host code; every computation happens in the kernels of gemm.hip, attention.hip and
// elementwise.hip, the same ones the encoder uses.
//
// Source: the Faster Transformer article (cloud.tencent.com/developer/article/1490359),
// section "什么是 Faster Transformer": decoder support is named there as a roadmap item; the
// layer read from it (the encoder layer plus a causal mask and a cross-attention
// sub-layer) is described in ftx_decoder.h.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "abi_common.h"
#include "ftx_decoder.h"
#include "launch.h"

using namespace ftx;

namespace {

struct DecLayerW {
  void *w_qkv_t, *b_qkv;    // [3H][H], [3H]: self-attention Q | K | V
  void *w_o_t, *b_o, *ln1_g, *ln1_b;
  void *w_q2_t, *b_q2;      // [H][H], [H]: cross-attention query
  void *w_kv2_t, *b_kv2;    // [2H][H], [2H]: cross-attention K | V over the memory
  void *w_o2_t, *b_o2, *ln2_g, *ln2_b;
  void *w1_t, *b1, *w2_t, *b2, *ln3_g, *ln3_b;
  void *w_qkvh_t, *b_qkvh;  // the self-attention Q | K | V rows ordered per head (Q_h, K_h,
                            // V_h), for the projection with the attention in its epilogue
};

}  // namespace

struct ftx_decoder {
  int B, Sd, Se, nh, d, L, H, F, Td, Tm;  // Sd, Se: internal lengths, multiples of 32;
                                          // Td = B Sd decoder rows, Tm = B Se memory rows
  int Sdv, Sev;                           // the caller's lengths (Sd, Se rounded up to 32)
  ftx_dtype dt;
  size_t es;
  int device;
  DeviceInfo dev;  // CU and XCD counts, read at create
  void* weights = nullptr;
  void* ws = nullptr;
  std::vector<DecLayerW> layers;
  std::vector<char> ready;
  // workspace views
  void *q, *k, *vt;      // self-attention [B][n][Sd][d], [B][n][Sd][d], [B][n][d][Sd]
  void *q2, *k2, *vt2;   // cross-attention [B][n][Sd][d], [B][n][Se][d], [B][n][d][Se]
  void *ctx, *abuf, *y1, *y2, *u;
  float* y1f = nullptr;  // fp32 copies of Y1 and Y2, the residuals of LayerNorms 2 and 3
  float* y2f = nullptr;  // (bf16 only)
  float* splitk = nullptr;
  size_t splitk_elems = 0;
  // when a caller length is not a multiple of 32: [B][Sd][H] input copy and layer state,
  // [B][Se][H] memory copy, their padding rows zero
  void *xpad = nullptr, *spad = nullptr, *mpad = nullptr;
  int timing = 0;
  int fused_attention = 1;  // 0 off, 1 from 256 rows and 64 tiles, 2 whenever the shape fits
  bool attn_fits = false;   // the per-head weight copy exists (qkv_attention_fits)
  struct Mark {
    hipEvent_t start, stop;
    int step;
  };
  std::vector<Mark> marks;       // recorded, not yet read
  std::vector<hipEvent_t> pool;  // free events
};

namespace {

ftx_status take_event(ftx_decoder* e, hipEvent_t* ev) {
  if (!e->pool.empty()) {
    *ev = e->pool.back();
    e->pool.pop_back();
    return FTX_OK;
  }
  FTX_HIP(hipEventCreate(ev));
  return FTX_OK;
}

// One launch, with an event pair around it on `s` when timing is on.
template <typename F>
ftx_status step(ftx_decoder* e, int cls, hipStream_t s, F&& launch) {
  ftx_decoder::Mark m{nullptr, nullptr, cls};
  if (e->timing) {
    ftx_status st = take_event(e, &m.start);
    if (st == FTX_OK) st = take_event(e, &m.stop);
    if (st != FTX_OK) return st;
    FTX_HIP(hipEventRecord(m.start, s));
  }
  const hipError_t err = launch();
  if (err != hipSuccess) return hip_fail(err, "kernel launch");
  if (e->timing) {
    FTX_HIP(hipEventRecord(m.stop, s));
    e->marks.push_back(m);
  }
  return FTX_OK;
}

// The causal self-attention runs inside the self Q/K/V projection when the shape fits and,
// in the default mode, under the encoder's rule (at least 256 decoder rows and a quarter as
// many 256-row tiles as the device has CUs).
bool use_fused_self_attention(const ftx_decoder* e) {
  if (!e->attn_fits || e->fused_attention == 0) return false;
  if (e->fused_attention == 2) return true;
  return fused_attention_pays(e->Td, e->H, e->dev.cus);
}

ftx_status enqueue_decoder(ftx_decoder* e, const void* input, const void* memory,
                           const int32_t* mem_lens, void* output, hipStream_t s) {
  const ftx_dtype dt = e->dt;
  const int B = e->B, Sd = e->Sd, Se = e->Se, nh = e->nh, d = e->d, H = e->H, F = e->F,
            Td = e->Td;
  const bool f32res = e->y1f != nullptr;
  float* ws = e->splitk;
  const size_t wn = e->splitk_elems;
  ftx_status st;
  // Projection a w_t (K = kin, N = H) and the add & LayerNorm after it: y = LN(xr + a w_t +
  // bias) (xr read as fp32 when xr_f32), yf an fp32 copy.  A projection that splits K (small
  // batches) leaves its fp32 partials to the LayerNorm, which sums them itself.
  auto proj_ln = [&](int proj_step, int ln_step, const void* a, const void* w_t, int kin,
                     const void* xr, bool xr_f32, const void* bias, const void* gamma,
                     const void* beta, void* y, float* yf) -> ftx_status {
    const int sp = linear_splits(dt, Td, H, kin, wn, true);
    ftx_status r;
    if (sp > 1) {
      if ((r = step(e, proj_step, s, [&] {
             return launch_linear_partials(dt, Td, H, kin, a, w_t, ws, wn, s);
           })) != FTX_OK) return r;
      return step(e, ln_step, s, [&] {
        return launch_splitk_bias_residual_layernorm(dt, Td, H, xr, xr_f32, ws, sp, f32res, bias,
                                                     gamma, beta, y, yf, s);
      });
    }
    if ((r = step(e, proj_step, s, [&] {
           return launch_linear(dt, Td, H, kin, a, w_t, nullptr, false, e->abuf, s, f32res, ws, wn);
         })) != FTX_OK) return r;
    return step(e, ln_step, s, [&] {
      return f32res ? launch_bias_residual_layernorm_f32res(dt, Td, H, xr, xr_f32, (const float*)e->abuf,
                                                            bias, gamma, beta, y, yf, s)
                    : launch_bias_residual_layernorm(dt, Td, H, xr, e->abuf, bias, gamma, beta, y, s);
    });
  };
  // Caller lengths below the internal ones: rows 0..Sdv-1 (0..Sev-1) of each sequence go to
  // the padded copies, the layers run at Sd and Se, and rows 0..Sdv-1 come back at the end.
  // Padded decoder rows follow the valid ones, so the causal mask keeps them out of every
  // valid row; padded memory rows are beyond the key range the cross-attention is limited to.
  const size_t row = (size_t)H * e->es;
  void* state = output;
  if (e->xpad) {
    FTX_HIP(hipMemcpy2DAsync(e->xpad, Sd * row, input, e->Sdv * row, e->Sdv * row, B,
                             hipMemcpyDeviceToDevice, s));
    input = e->xpad;
    state = e->spad;
  }
  if (e->mpad) {
    FTX_HIP(hipMemcpy2DAsync(e->mpad, Se * row, memory, e->Sev * row, e->Sev * row, B,
                             hipMemcpyDeviceToDevice, s));
    memory = e->mpad;
  }
  for (int l = 0; l < e->L; ++l) {
    const DecLayerW& w = e->layers[l];
    const void* x = l == 0 ? input : state;
    // causal self-attention, add & LayerNorm 1
    if (use_fused_self_attention(e)) {
      if ((st = step(e, FTX_DEC_STEP_SELF_QKV_ATTENTION, s, [&] {
             return launch_qkv_attention(dt, B, Sd, nh, d, x, w.w_qkvh_t, w.b_qkvh, nullptr, Sd,
                                         e->ctx, s, true);
           })) != FTX_OK) return st;
    } else {
      if ((st = step(e, FTX_DEC_STEP_SELF_QKV_GEMM, s, [&] {
             return launch_qkv_projection(dt, B, Sd, nh, d, x, w.w_qkv_t, w.b_qkv, e->q, e->k,
                                          e->vt, s, ws, wn);
           })) != FTX_OK) return st;
      if ((st = step(e, FTX_DEC_STEP_SELF_ATTENTION, s, [&] {
             return launch_attention(dt, B, Sd, Sd, nh, d, e->q, e->k, e->vt, nullptr, e->ctx, s,
                                     Sd, true);
           })) != FTX_OK) return st;
    }
    if ((st = proj_ln(FTX_DEC_STEP_SELF_OUT_GEMM, FTX_DEC_STEP_LN1, e->ctx, w.w_o_t, H, x, false,
                      w.b_o, w.ln1_g, w.ln1_b, e->y1, e->y1f)) != FTX_OK) return st;
    // cross-attention over the memory, add & LayerNorm 2
    if ((st = step(e, FTX_DEC_STEP_CROSS_Q_GEMM, s, [&] {
           return launch_head_projection(dt, B, Sd, nh, d, e->y1, w.w_q2_t, w.b_q2, 0, 1, e->q2,
                                         nullptr, nullptr, s, ws, wn);
         })) != FTX_OK) return st;
    if ((st = step(e, FTX_DEC_STEP_CROSS_KV_GEMM, s, [&] {
           return launch_head_projection(dt, B, Se, nh, d, memory, w.w_kv2_t, w.b_kv2, 1, 2,
                                         nullptr, e->k2, e->vt2, s, ws, wn);
         })) != FTX_OK) return st;
    if ((st = step(e, FTX_DEC_STEP_CROSS_ATTENTION, s, [&] {
           return launch_attention(dt, B, Sd, Se, nh, d, e->q2, e->k2, e->vt2, mem_lens, e->ctx, s,
                                   e->Sev, false);
         })) != FTX_OK) return st;
    if ((st = proj_ln(FTX_DEC_STEP_CROSS_OUT_GEMM, FTX_DEC_STEP_LN2, e->ctx, w.w_o2_t, H,
                      f32res ? (const void*)e->y1f : e->y1, f32res, w.b_o2, w.ln2_g, w.ln2_b,
                      e->y2, e->y2f)) != FTX_OK) return st;
    // feed-forward, add & LayerNorm 3 (written to the output, the next layer's input)
    if ((st = step(e, FTX_DEC_STEP_FFN1_GEMM, s, [&] {
           return launch_linear(dt, Td, F, H, e->y2, w.w1_t, w.b1, true, e->u, s, false, ws, wn);
         })) != FTX_OK) return st;
    if ((st = proj_ln(FTX_DEC_STEP_FFN2_GEMM, FTX_DEC_STEP_LN3, e->u, w.w2_t, F,
                      f32res ? (const void*)e->y2f : e->y2, f32res, w.b2, w.ln3_g, w.ln3_b, state,
                      nullptr)) != FTX_OK) return st;
  }
  if (e->xpad)
    FTX_HIP(hipMemcpy2DAsync(output, e->Sdv * row, state, Sd * row, e->Sdv * row, B,
                             hipMemcpyDeviceToDevice, s));
  return FTX_OK;
}

}  // namespace

extern "C" {

ftx_status ftx_decoder_create(int batch_size, int tgt_len, int mem_len, int head_num,
                              int size_per_head, int num_layers, ftx_dtype dtype,
                              ftx_decoder** out) {
  last_error_slot().clear();
  if (!out) return fail(FTX_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!dtype_ok(dtype)) return fail(FTX_ERR_INVALID_ARG, "unknown dtype");
  if (num_layers < 1) return fail(FTX_ERR_INVALID_ARG, "num_layers must be >= 1");
  ftx_status st = check_shape(batch_size, tgt_len, head_num, size_per_head, true);
  if (st == FTX_OK) st = check_shape(batch_size, mem_len, head_num, size_per_head, true);
  if (st != FTX_OK) return st;

  int dev = 0;
  FTX_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  FTX_HIP(hipGetDeviceProperties(&prop, dev));
  if (std::string(prop.gcnArchName).rfind("gfx950", 0) != 0)
    return fail(FTX_ERR_UNSUPPORTED, std::string("built for gfx950, device is ") + prop.gcnArchName);

  ftx_decoder* e = new (std::nothrow) ftx_decoder();
  if (!e) return fail(FTX_ERR_OUT_OF_MEMORY, "host allocation");
  e->B = batch_size;
  e->Sdv = tgt_len;
  e->Sev = mem_len;
  e->Sd = (tgt_len + 31) / 32 * 32;
  e->Se = (mem_len + 31) / 32 * 32;
  e->nh = head_num;
  e->d = size_per_head;
  e->L = num_layers;
  e->H = head_num * size_per_head;
  e->F = 4 * e->H;
  e->Td = batch_size * e->Sd;
  e->Tm = batch_size * e->Se;
  e->dt = dtype;
  e->es = dtype_size(dtype);
  e->device = dev;
  e->dev = device_info();

  const size_t H = e->H, F = e->F, Td = e->Td, Tm = e->Tm, es = e->es;
  auto pad = [](size_t bytes) { return (bytes + 255) / 256 * 256; };
  // per layer: Wqkv 3HH + 3H, Wo HH + H, LN1 2H, Wq2 HH + H, Wkv2 2HH + 2H, Wo2 HH + H,
  // LN2 2H, W1 FH + F, W2 HF + H, LN3 2H
  // (+ 3HH + 3H in per-head order when the fused self-attention fits)
  e->attn_fits = qkv_attention_fits(dtype, e->Sd, head_num, size_per_head);
  const size_t per_layer = pad(3 * H * H * es) + pad(3 * H * es) + 3 * pad(H * H * es) +
                           pad(2 * H * H * es) + pad(2 * H * es) + pad(F * H * es) + pad(F * es) +
                           pad(H * F * es) + 10 * pad(H * es) +
                           (e->attn_fits ? pad(3 * H * H * es) + pad(3 * H * es) : 0);
  hipError_t err = hipMalloc(&e->weights, per_layer * e->L);
  if (err != hipSuccess) {
    delete e;
    return hip_fail(err, "hipMalloc(weights)");
  }
  const bool f32res = dtype == FTX_BF16;
  const size_t TdH = pad(Td * H * es), TmH = pad(Tm * H * es), F32 = pad(Td * H * 4);
  const bool xpadded = e->Sdv != e->Sd, mpadded = e->Sev != e->Se;
  const size_t ws_bytes = 4 * TdH /*q,k,vt,q2*/ + 2 * TmH /*k2,vt2*/ + TdH /*ctx*/ +
                          (f32res ? F32 : TdH) /*abuf*/ + 2 * TdH /*y1,y2*/ +
                          pad(Td * F * es) /*u*/ + (f32res ? 2 * F32 : 0) /*y1f,y2f*/ +
                          (xpadded ? 2 * TdH : 0) /*xpad,spad*/ + (mpadded ? TmH : 0) /*mpad*/;
  err = hipMalloc(&e->ws, ws_bytes);
  if (err != hipSuccess) {
    hipFree(e->weights);
    delete e;
    return hip_fail(err, "hipMalloc(workspace)");
  }
  char* w = (char*)e->weights;
  e->layers.resize(e->L);
  for (int l = 0; l < e->L; ++l) {
    DecLayerW& lw = e->layers[l];
    auto take = [&](size_t bytes) { void* p = w; w += pad(bytes); return p; };
    lw.w_qkv_t = take(3 * H * H * es);
    lw.b_qkv = take(3 * H * es);
    lw.w_o_t = take(H * H * es);
    lw.b_o = take(H * es);
    lw.ln1_g = take(H * es);
    lw.ln1_b = take(H * es);
    lw.w_q2_t = take(H * H * es);
    lw.b_q2 = take(H * es);
    lw.w_kv2_t = take(2 * H * H * es);
    lw.b_kv2 = take(2 * H * es);
    lw.w_o2_t = take(H * H * es);
    lw.b_o2 = take(H * es);
    lw.ln2_g = take(H * es);
    lw.ln2_b = take(H * es);
    lw.w1_t = take(F * H * es);
    lw.b1 = take(F * es);
    lw.w2_t = take(H * F * es);
    lw.b2 = take(H * es);
    lw.ln3_g = take(H * es);
    lw.ln3_b = take(H * es);
    lw.w_qkvh_t = e->attn_fits ? take(3 * H * H * es) : nullptr;
    lw.b_qkvh = e->attn_fits ? take(3 * H * es) : nullptr;
  }
  e->ready.assign(e->L, 0);
  char* p = (char*)e->ws;
  e->q = p; p += TdH;
  e->k = p; p += TdH;
  e->vt = p; p += TdH;
  e->q2 = p; p += TdH;
  e->k2 = p; p += TmH;
  e->vt2 = p; p += TmH;
  e->ctx = p; p += TdH;
  e->abuf = p; p += f32res ? F32 : TdH;
  e->y1 = p; p += TdH;
  e->y2 = p; p += TdH;
  e->u = p; p += pad(Td * F * es);
  if (f32res) {
    e->y1f = (float*)p; p += F32;
    e->y2f = (float*)p; p += F32;
  }
  if (xpadded) {
    e->xpad = p; p += TdH;
    e->spad = p; p += TdH;
  }
  if (mpadded) {
    e->mpad = p; p += TmH;
  }
  if (xpadded || mpadded) {
    // padding rows of the copies stay zero (only rows below the caller's lengths are ever
    // written); the state's padding rows are computed and never reach a valid row
    hipError_t zerr = hipSuccess;
    if (xpadded) zerr = hipMemset(e->xpad, 0, 2 * TdH);
    if (zerr == hipSuccess && mpadded) zerr = hipMemset(e->mpad, 0, TmH);
    if (zerr == hipSuccess) zerr = hipDeviceSynchronize();
    if (zerr != hipSuccess) {
      hipFree(e->ws);
      hipFree(e->weights);
      delete e;
      return hip_fail(zerr, "hipMemset(padding)");
    }
  }
  // split-K workspace: the largest any of the six projections plans for
  const int Tdi = e->Td, Tmi = e->Tm, Hi = e->H, Fi = e->F;
  const size_t need = std::max({gemm_splitk_workspace(dtype, Tdi, 3 * Hi, Hi),
                                gemm_splitk_workspace(dtype, Tdi, Hi, Hi),
                                gemm_splitk_workspace(dtype, Tmi, 2 * Hi, Hi),
                                gemm_splitk_workspace(dtype, Tdi, Fi, Hi),
                                gemm_splitk_workspace(dtype, Tdi, Hi, Fi)});
  if (need) {
    err = hipMalloc(&e->splitk, need * sizeof(float));
    if (err != hipSuccess) {
      hipFree(e->ws);
      hipFree(e->weights);
      delete e;
      return hip_fail(err, "hipMalloc(split-K workspace)");
    }
    e->splitk_elems = need;
  }
  *out = e;
  return FTX_OK;
}

ftx_status ftx_decoder_set_weights(ftx_decoder* e, int layer, const ftx_decoder_layer_weights* w,
                                   void* stream) {
  last_error_slot().clear();
  if (!e) return fail(FTX_ERR_INVALID_ARG, "decoder is NULL");
  if (!w) return fail(FTX_ERR_INVALID_ARG, "weights struct is NULL");
  if (layer < 0 || layer >= e->L) return fail(FTX_ERR_INVALID_ARG, "layer out of range");
  const void* ptrs[] = {w->w_q,  w->b_q,  w->w_k,  w->b_k,  w->w_v,  w->b_v,  w->w_o,
                        w->b_o,  w->ln1_gamma, w->ln1_beta, w->w_q2, w->b_q2, w->w_k2,
                        w->b_k2, w->w_v2, w->b_v2, w->w_o2, w->b_o2, w->ln2_gamma,
                        w->ln2_beta, w->w_ffn1, w->b_ffn1, w->w_ffn2, w->b_ffn2,
                        w->ln3_gamma, w->ln3_beta};
  for (const void* p : ptrs)
    if (!p) return fail(FTX_ERR_INVALID_ARG, "a weight pointer is NULL");
  for (const void* p : ptrs)
    if (!is_device_ptr(p)) return fail(FTX_ERR_INVALID_ARG, "a weight pointer is not device memory");
  hipStream_t s = (hipStream_t)stream;
  FTX_HIP(hipSetDevice(e->device));
  const int Hi = e->H, Fi = e->F;
  const size_t H = e->H, F = e->F, es = e->es, HH = H * H * es;
  DecLayerW& lw = e->layers[layer];
  // matrices stored transposed [out][in]; Q|K|V and K2|V2 stacked along out
  char* qkv = (char*)lw.w_qkv_t;
  FTX_HIP(launch_transpose(e->dt, Hi, Hi, w->w_q, qkv, s));
  FTX_HIP(launch_transpose(e->dt, Hi, Hi, w->w_k, qkv + HH, s));
  FTX_HIP(launch_transpose(e->dt, Hi, Hi, w->w_v, qkv + 2 * HH, s));
  FTX_HIP(launch_transpose(e->dt, Hi, Hi, w->w_o, lw.w_o_t, s));
  FTX_HIP(launch_transpose(e->dt, Hi, Hi, w->w_q2, lw.w_q2_t, s));
  char* kv2 = (char*)lw.w_kv2_t;
  FTX_HIP(launch_transpose(e->dt, Hi, Hi, w->w_k2, kv2, s));
  FTX_HIP(launch_transpose(e->dt, Hi, Hi, w->w_v2, kv2 + HH, s));
  FTX_HIP(launch_transpose(e->dt, Hi, Hi, w->w_o2, lw.w_o2_t, s));
  FTX_HIP(launch_transpose(e->dt, Hi, Fi, w->w_ffn1, lw.w1_t, s));
  FTX_HIP(launch_transpose(e->dt, Fi, Hi, w->w_ffn2, lw.w2_t, s));
  auto copy = [&](void* dst, const void* src, size_t n) {
    return hipMemcpyAsync(dst, src, n * es, hipMemcpyDeviceToDevice, s);
  };
  char* bqkv = (char*)lw.b_qkv;
  char* bkv2 = (char*)lw.b_kv2;
  FTX_HIP(copy(bqkv, w->b_q, H));
  FTX_HIP(copy(bqkv + H * es, w->b_k, H));
  FTX_HIP(copy(bqkv + 2 * H * es, w->b_v, H));
  FTX_HIP(copy(lw.b_o, w->b_o, H));
  FTX_HIP(copy(lw.ln1_g, w->ln1_gamma, H));
  FTX_HIP(copy(lw.ln1_b, w->ln1_beta, H));
  FTX_HIP(copy(lw.b_q2, w->b_q2, H));
  FTX_HIP(copy(bkv2, w->b_k2, H));
  FTX_HIP(copy(bkv2 + H * es, w->b_v2, H));
  FTX_HIP(copy(lw.b_o2, w->b_o2, H));
  FTX_HIP(copy(lw.ln2_g, w->ln2_gamma, H));
  FTX_HIP(copy(lw.ln2_b, w->ln2_beta, H));
  FTX_HIP(copy(lw.b1, w->b_ffn1, F));
  FTX_HIP(copy(lw.b2, w->b_ffn2, H));
  FTX_HIP(copy(lw.ln3_g, w->ln3_gamma, H));
  FTX_HIP(copy(lw.ln3_b, w->ln3_beta, H));
  if (lw.w_qkvh_t) {
    // rows of head h of Q (K, V) go to rows 3 d h .. (+d, +2d)
    const size_t d = e->d;
    for (int part = 0; part < 3; ++part) {
      FTX_HIP(hipMemcpy2DAsync((char*)lw.w_qkvh_t + part * d * H * es, 3 * d * H * es,
                               qkv + part * HH, d * H * es, d * H * es, e->nh,
                               hipMemcpyDeviceToDevice, s));
      FTX_HIP(hipMemcpy2DAsync((char*)lw.b_qkvh + part * d * es, 3 * d * es, bqkv + part * H * es,
                               d * es, d * es, e->nh, hipMemcpyDeviceToDevice, s));
    }
  }
  FTX_HIP(hipStreamSynchronize(s));
  e->ready[layer] = 1;
  return FTX_OK;
}

ftx_status ftx_decoder_forward(ftx_decoder* e, const void* input, const void* memory,
                               const int32_t* mem_lens, void* output, void* stream) {
  last_error_slot().clear();
  if (!e) return fail(FTX_ERR_INVALID_ARG, "decoder is NULL");
  if (!input || !memory || !output) return fail(FTX_ERR_INVALID_ARG, "input, memory or output is NULL");
  if (!aligned16(input) || !aligned16(memory) || !aligned16(output))
    return fail(FTX_ERR_INVALID_ARG, "input, memory and output must be 16-byte aligned");
  const size_t xb = (size_t)e->B * e->Sdv * e->H * e->es, mb = (size_t)e->B * e->Sev * e->H * e->es;
  if (overlap(input, xb, output, xb) || overlap(memory, mb, output, xb))
    return fail(FTX_ERR_INVALID_ARG, "output overlaps input or memory");
  for (int l = 0; l < e->L; ++l)
    if (!e->ready[l]) return fail(FTX_ERR_NOT_READY, "layer " + std::to_string(l) + " has no weights");
  if (!all_device({input, memory, output, mem_lens}))
    return fail(FTX_ERR_INVALID_ARG, "input, memory, output and mem_lens must be device memory");
  FTX_HIP(hipSetDevice(e->device));
  return enqueue_decoder(e, input, memory, mem_lens, output, (hipStream_t)stream);
}

ftx_status ftx_decoder_set_option(ftx_decoder* e, ftx_option option, int value) {
  last_error_slot().clear();
  if (!e) return fail(FTX_ERR_INVALID_ARG, "decoder is NULL");
  if (option == FTX_OPT_KERNEL_TIMING) {
    e->timing = value ? 1 : 0;
    return FTX_OK;
  }
  if (option == FTX_OPT_FUSED_ATTENTION) {
    if (value < 0 || value > 2) return fail(FTX_ERR_INVALID_ARG, "fused attention mode is 0, 1 or 2");
    e->fused_attention = value;
    return FTX_OK;
  }
  return fail(FTX_ERR_INVALID_ARG, "option not available for the decoder");
}

ftx_status ftx_decoder_kernel_times(ftx_decoder* e, double* ms, int64_t* counts) {
  last_error_slot().clear();
  if (!e) return fail(FTX_ERR_INVALID_ARG, "decoder is NULL");
  double acc[FTX_DEC_NUM_STEPS] = {0};
  int64_t cnt[FTX_DEC_NUM_STEPS] = {0};
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
  for (int i = 0; i < FTX_DEC_NUM_STEPS; ++i) {
    if (ms) ms[i] = acc[i];
    if (counts) counts[i] = cnt[i];
  }
  return FTX_OK;
}

ftx_status ftx_decoder_destroy(ftx_decoder* e) {
  last_error_slot().clear();
  if (!e) return FTX_OK;
  hipSetDevice(e->device);
  hipDeviceSynchronize();
  for (auto& m : e->marks) {
    hipEventDestroy(m.start);
    hipEventDestroy(m.stop);
  }
  for (auto ev : e->pool) hipEventDestroy(ev);
  if (e->splitk) hipFree(e->splitk);
  hipFree(e->weights);
  hipFree(e->ws);
  delete e;
  return FTX_OK;
}

}  // extern "C"
