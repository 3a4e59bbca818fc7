// Fused multi-head self-attention of the encoder layer on CDNA4 matrix cores.
//
// Source: the Faster Transformer article (cloud.tencent.com/developer/article/1490359),
// section "Faster Transformer 优化原理": per layer, the batched Q K^T and P V matrix
// multiplies with a SoftMax kernel between them (two SoftMax versions chosen by shape,
// row sums by register shuffle, sums kept in float), plus the transposes around them.
// Here the whole chain for one (sequence, head, 32-query block) runs in one wavefront,
// with K and V^T of the head shared by the workgroup through LDS:
//
//   S^T = K Q^T       v_mfma 32x32 tiles, keys on rows, the wave's 32 queries on columns;
//                     a lane then holds 16 of the 32 keys of one query per tile;
//   mask, scale       keys j >= len_b get -inf (only tiles reaching len_b are masked key by
//                     key); scores scaled by 1/sqrt(d) inside the hardware exp2;
//   softmax           row max and sum: the lane's own values, then one cross-lane step
//                     (lane ^ 32, a register swap of the wave's halves) -- the wave64
//                     form of the shuffle row reduction; fp32;
//   C^T = V^T P^T     the probabilities stay in registers and are fed, converted to the
//                     storage type, straight into the next MFMA as its B operand; V is
//                     read from the per-head transposed layout V^T[d][S];
//   merge heads       the result is staged in LDS and stored at ctx[b*S + i][h*d + e].
// (For S = 32 with few heads in flight a variant without LDS reads every operand straight
// from global memory; see attention_s32_kernel.)
//
// Key tiles are processed in chunks of up to 4 (128 keys) with the running-max
// rescaling of the streaming softmax, so S = 512 uses the same kernel; for S <= 128 the
// loop runs once.  Key tiles entirely beyond len_b are neither loaded nor multiplied:
// their probabilities are exactly 0.  Every query row, padded or not, is computed.
// 16-bit data takes attention_dma_kernel: four query blocks per workgroup, operands loaded
// into LDS without passing through registers, K and V^T streamed through a two-chunk ring
// so that two or three workgroups share a CU; fp32 takes attention_kernel.

#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace ftx {

template <typename T> struct AttnMfma;

// sum(a) adds the elements of a probability fragment to acc: two at a time with the
// packed dot product against (1, 1) for 16-bit data (the very values the next MFMA uses).
template <> struct AttnMfma<f16> {
  static constexpr int VEC = 8;
  typedef f16x8 frag;
  typedef _Float16 pair __attribute__((ext_vector_type(2)));
  __device__ static __forceinline__ void mma(const frag& a, const frag& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float sum(const frag& a, float acc) {
    const pair one = {(f16)1.0f, (f16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2(pair{a[2 * i], a[2 * i + 1]}, one, acc, false);
    return acc;
  }
};
template <> struct AttnMfma<bf16> {
  static constexpr int VEC = 8;
  typedef bf16x8 frag;
  typedef __bf16 pair __attribute__((ext_vector_type(2)));
  __device__ static __forceinline__ void mma(const frag& a, const frag& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float sum(const frag& a, float acc) {
    const pair one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(pair{a[2 * i], a[2 * i + 1]}, one, acc, false);
    return acc;
  }
};
template <> struct AttnMfma<float> {
  static constexpr int VEC = 4;  // one 16-byte fragment feeds four 32x32x2 steps
  typedef f32x4 frag;
  __device__ static __forceinline__ void mma(const frag& a, const frag& b, f32x16& c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  }
  __device__ static __forceinline__ float sum(const frag& a, float acc) {
    return acc + ((a[0] + a[1]) + (a[2] + a[3]));
  }
};

// Fallback for shapes whose K and V^T do not fit in LDS (fp32 with d = 64 and S > 256):
// the same chain with every wave reading its head's K and V^T straight from global
// memory, and the output stored from registers.
template <typename T, int D>
__global__ __launch_bounds__(256) void attention_global_kernel(const T* __restrict__ q,
                                                        const T* __restrict__ k,
                                                        const T* __restrict__ vt,
                                                        const int32_t* __restrict__ lens,
                                                        T* __restrict__ ctx, int B, int Sq, int Sk,
                                                        int nh, float scale_log2e, int s_valid,
                                                        int causal) {
  typedef AttnMfma<T> MF;
  typedef typename MF::frag frag;
  typedef typename VecT<T, 4>::type v4;
  constexpr int VEC = MF::VEC;
  constexpr int KF = 2 * VEC;   // d consumed per fragment pair
  constexpr int NQF = D / KF;   // fragments along d
  constexpr int DT = D / 32;    // 32-row tiles of the transposed output along d
  constexpr int CH = 4;         // key tiles per softmax chunk
  constexpr int WPB = 4;        // waves per block

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lr = lane % 32, g = lane / 32;
  const int qblocks = Sq / 32;
  const int ntasks = B * nh * qblocks;
  // hand each XCD a contiguous range of tasks so the waves reading one head's K and V
  // share that XCD's L2
  const int nblk = gridDim.x;
  int blk = blockIdx.x;
  if (nblk % 8 == 0) blk = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
  const int task = blk * WPB + wave;
  if (task >= ntasks) return;
  const int bh = task / qblocks, qb = task % qblocks;
  const int b = bh / nh, h = bh % nh;
  int len = lens ? lens[b] : s_valid;
  len = min(max(len, 1), s_valid);
  int nkt = (len + 31) / 32;
  if (causal) nkt = min(nkt, qb + 1);  // later key tiles are entirely in the future
  const int query = qb * 32 + lr;

  frag qf[NQF];
  {
    const T* qp = q + ((size_t)bh * Sq + qb * 32 + lr) * D + g * VEC;
#pragma unroll
    for (int f = 0; f < NQF; ++f) qf[f] = *(const frag*)(qp + f * KF);
  }
  const T* kbase = k + (size_t)bh * Sk * D + g * VEC;
  const T* vbase = vt + (size_t)bh * D * Sk;

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int c0 = 0; c0 < nkt; c0 += CH) {
    f32x16 sc[CH];
#pragma unroll
    for (int t = 0; t < CH; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
      const int kt = c0 + t;
      if (kt < nkt) {
        const T* kr = kbase + (size_t)(kt * 32 + lr) * D;
#pragma unroll
        for (int f = 0; f < NQF; ++f) MF::mma(*(const frag*)(kr + f * KF), qf[f], sc[t]);
      }
    }
    // mask and chunk maximum (key of register r: tile*32 + 8*(r/4) + 4*g + r%4); only a key
    // tile that reaches the valid length or (causal) the query block's diagonal needs the
    // per-key mask
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const int kb = (c0 + t) * 32;
      if (kb + 32 > len || (causal && kb + 31 > qb * 32)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 8 * (r / 4) + 4 * g + (r % 4);
          if (key >= len || (causal && key > query)) sc[t][r] = -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);  // finite: the first chunk holds key 0 < len
    const float alpha = exp2_flush((m_run - m_new) * scale_log2e);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < CH; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_flush((sc[t][r] - m_new) * scale_log2e);
        sc[t][r] = p;
        psum += p;
      }
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

    // context: o[dt] += V^T[dt tile][keys] * P^T[keys][queries]
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const int kt = c0 + t;
      if (kt >= nkt) continue;
      if constexpr (VEC == 8) {
        // MFMA u consumes P registers 8u..8u+7 = keys kt*32 + 16u + {0..3, 8..11} + 4g
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          frag pf;
#pragma unroll
          for (int s = 0; s < 8; ++s) pf[s] = from_f32<T>(sc[t][8 * u + s]);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const T* vr = vbase + (size_t)(dt * 32 + lr) * Sk + kt * 32 + 16 * u + 4 * g;
            const v4 lo = *(const v4*)(vr);
            const v4 hi = *(const v4*)(vr + 8);
            frag vf;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              vf[s] = lo[s];
              vf[s + 4] = hi[s];
            }
            MF::mma(vf, pf, o[dt]);
          }
        }
      } else {
        // fp32: call u consumes registers 4u..4u+3 = keys kt*32 + 8u + 4g + {0..3}
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          frag pf;
#pragma unroll
          for (int s = 0; s < 4; ++s) pf[s] = sc[t][4 * u + s];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const T* vr = vbase + (size_t)(dt * 32 + lr) * Sk + kt * 32 + 8 * u + 4 * g;
            MF::mma(*(const frag*)vr, pf, o[dt]);
          }
        }
      }
    }
  }

  // normalise and store with heads merged: ctx[b*Sq + query][h*D + dd]
  const float inv = 1.0f / l_run;
  const int H = nh * D;
  T* out = ctx + ((size_t)b * Sq + qb * 32 + lr) * H + h * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      v4 vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = from_f32<T>(o[dt][4 * rr + e] * inv);
      *(v4*)(out + dt * 32 + 8 * rr) = vv;
    }
}


// One workgroup per (sequence, head, group of up to 8 query blocks of 32).  The workgroup
// first copies K [keys][d] and V^T [d][keys] of its head -- only the key tiles below the
// sequence's valid length -- into row-padded LDS with 16-byte coalesced loads; every wave
// then reads its MFMA fragments from LDS, so K and V leave HBM once per workgroup instead
// of once per wave.  At the end the waves stage their context tiles in LDS (rows of d) and
// store whole 2*D-byte rows of the merged-heads output with 16-byte vectors.
template <typename T, int D, int SMAX> struct AttnCfg {
  static constexpr int VE = 16 / sizeof(T);          // elements per 16-byte vector
  static constexpr int NW = SMAX / 32 < 8 ? SMAX / 32 : 8;  // waves per workgroup
  static constexpr int CH = SMAX / 32 < 4 ? SMAX / 32 : 4;  // key tiles per softmax chunk
  static constexpr int KST = D + VE;                 // LDS row stride of K (elements)
  static constexpr int VST = SMAX + VE;              // LDS row stride of V^T
  static constexpr int OST = D + VE;                 // LDS row stride of the output stage
  static constexpr int LDS = SMAX * KST + D * VST;   // elements
  static_assert(NW * 32 * OST <= LDS, "output stage must fit in the K/V area");
};

template <typename T, int D, int SMAX>
__global__ __launch_bounds__((AttnCfg<T, D, SMAX>::NW * kWave)) void attention_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ vt,
    const int32_t* __restrict__ lens, T* __restrict__ ctx, int B, int Sq, int Sk, int nh,
    float scale_log2e, int s_valid, int causal, int xcds) {
  typedef AttnCfg<T, D, SMAX> C;
  typedef AttnMfma<T> MF;
  typedef typename MF::frag frag;
  typedef typename VecT<T, 4>::type v4;
  typedef typename Vec16<T>::type vec;
  constexpr int VEC = MF::VEC;
  constexpr int KF = 2 * VEC;   // d consumed per fragment pair
  constexpr int NQF = D / KF;   // fragments along d
  constexpr int DT = D / 32;    // 32-row tiles of the transposed output along d
  constexpr int CH = C::CH;     // key tiles per softmax chunk
  constexpr int NT = C::NW * kWave;
  __shared__ __attribute__((aligned(16))) T smem[C::LDS];
  T* Ks = smem;
  T* Vs = smem + SMAX * C::KST;

  const int qblocks = Sq / 32;
  const int groups = (qblocks + C::NW - 1) / C::NW;
  int blk = blockIdx.x;
  if (groups > 1 && xcds > 1 && (B * nh) % xcds == 0) {
    // workgroups go to the XCDs round-robin; renumber them so that the query groups of one
    // head run side by side on one XCD and its L2 serves the K/V^T reads after the first
    const int x = blk % xcds, slot = blk / xcds;
    blk = ((slot / groups) * xcds + x) * groups + slot % groups;
  }
  const int bh = blk / groups, grp = blk % groups;
  const int b = bh / nh, h = bh % nh;
  // the wave index is the same in every lane of a wave; stating it keeps the query block,
  // the key-tile counts and every per-tile test below in scalar registers and branches
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 32, g = lane / 32;
  const int qb = grp * C::NW + wave;
  const bool active = qb < qblocks;
  int len = lens ? lens[b] : s_valid;
  len = min(max(len, 1), s_valid);
  int nkt = (len + 31) / 32;       // key tiles of this wave
  int nk = nkt * 32;               // keys held in LDS (for every wave of the group)
  int clean = len / 32;            // leading key tiles that need no per-key mask
  if (causal) {
    // key tiles after a query block are entirely in its future
    nk = min(nkt, min(grp * C::NW + C::NW, qblocks)) * 32;
    nkt = min(nkt, qb + 1);
    clean = min(clean, qb);
  }
  const int query = qb * 32 + lr;

  frag qf[NQF];
  if (active) {
    const T* qp = q + ((size_t)bh * Sq + qb * 32 + lr) * D + g * VEC;
#pragma unroll
    for (int f = 0; f < NQF; ++f) qf[f] = *(const frag*)(qp + f * KF);
  }
  {
    // K rows and V^T columns below nk, as 16-byte vectors; the loops run to the
    // compile-time maximum with a per-vector predicate, so every load of a thread is issued
    // before its first LDS store
    constexpr int KCH = D / C::VE;                   // vectors per K row
    constexpr int KPT = (SMAX * KCH + NT - 1) / NT;  // K vectors per thread
    constexpr int VCH = SMAX / C::VE;                // vectors per V^T row
    constexpr int VPT = (D * VCH + NT - 1) / NT;
    const T* kg = k + (size_t)bh * Sk * D;
    const T* vg = vt + (size_t)bh * D * Sk;
    vec kb[KPT], vb[VPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = threadIdx.x + i * NT, r = c / KCH;
      if (c < SMAX * KCH && r < nk) kb[i] = *(const vec*)(kg + (size_t)r * D + (c % KCH) * C::VE);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * NT, col = (c % VCH) * C::VE;
      if (c < D * VCH && col < nk) vb[i] = *(const vec*)(vg + (size_t)(c / VCH) * Sk + col);
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = threadIdx.x + i * NT, r = c / KCH;
      if (c < SMAX * KCH && r < nk) *(vec*)(Ks + r * C::KST + (c % KCH) * C::VE) = kb[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * NT, col = (c % VCH) * C::VE;
      if (c < D * VCH && col < nk) *(vec*)(Vs + (c / VCH) * C::VST + col) = vb[i];
    }
  }
  __syncthreads();

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float l_run = 1.f;

  if (active) {
    constexpr int NU = 16 / VEC;   // probability fragments per 32-key tile
    float m_run = -INFINITY;
    l_run = 0.f;
    const T* kbase = Ks + lr * C::KST + g * VEC;
    const T* vbase = Vs + lr * C::VST + 4 * g;
    // One chunk of CH key tiles from tile c0.  Chunks below `clean` run without a single
    // test; the tail chunk skips tiles past nkt (their probabilities are set to exactly 0)
    // and masks keys key by key where a tile reaches len_b or the causal diagonal.
    auto chunk = [&](const int c0, auto tail) {
      constexpr bool TAIL = decltype(tail)::value;
      f32x16 sc[CH];
#pragma unroll
      for (int t = 0; t < CH; ++t) {
        if (!TAIL || c0 + t < nkt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
          const T* kr = kbase + (c0 + t) * 32 * C::KST;
#pragma unroll
          for (int f = 0; f < NQF; ++f) MF::mma(*(const frag*)(kr + f * KF), qf[f], sc[t]);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[t][r] = -INFINITY;
        }
      }
      if constexpr (TAIL) {
        // key of register r: tile*32 + 8*(r/4) + 4*g + r%4
#pragma unroll
        for (int t = 0; t < CH; ++t) {
          const int kb = (c0 + t) * 32;
          if (c0 + t < nkt && (kb + 32 > len || (causal && kb + 31 > qb * 32))) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb + 8 * (r / 4) + 4 * g + (r % 4);
              if (key >= len || (causal && key > query)) sc[t][r] = -INFINITY;
            }
          }
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < CH; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
      // finite: every chunk's first key is below len and (causal) not after the query
      const float m_new = fmaxf(m_run, fmaxf(mx, half_swap(mx)));
      const float mc = m_new * scale_log2e;
      const float alpha = exp2_flush(fmaf(m_run, scale_log2e, -mc));  // 0 on the first chunk
      m_run = m_new;
      // probabilities in the storage type, as the next MFMA's B operand: fragment u of a
      // tile holds registers VEC*u .. VEC*u + VEC-1; the row sum adds exactly these values
      frag pf[CH][NU];
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < CH; ++t)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
          for (int e = 0; e < VEC; ++e)
            pf[t][u][e] = from_f32<T>(exp2_flush(fmaf(sc[t][VEC * u + e], scale_log2e, -mc)));
          psum = MF::sum(pf[t][u], psum);
        }
      l_run = l_run * alpha + (psum + half_swap(psum));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

      // context: o[dt] += V^T[dt tile][keys] * P^T[keys][queries]; fragment u takes keys
      // tile*32 + 2*VEC*u + 4g + {0..3} (and + 8 + {0..3} for 16-bit data)
#pragma unroll
      for (int t = 0; t < CH; ++t) {
        if (TAIL && c0 + t >= nkt) continue;
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const T* vr = vbase + dt * 32 * C::VST + (c0 + t) * 32 + 2 * VEC * u;
            if constexpr (VEC == 8) {
              const v4 lo = *(const v4*)(vr);
              const v4 hi = *(const v4*)(vr + 8);
              frag vf;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                vf[e] = lo[e];
                vf[e + 4] = hi[e];
              }
              MF::mma(vf, pf[t][u], o[dt]);
            } else {
              MF::mma(*(const frag*)vr, pf[t][u], o[dt]);
            }
          }
      }
    };
    int c0 = 0;
    for (; c0 + CH <= clean; c0 += CH) chunk(c0, std::false_type{});
    for (; c0 < nkt; c0 += CH) chunk(c0, std::true_type{});
  }

  // normalise, stage [query][d] in LDS (the K/V area is free once every wave is past here),
  // then store whole rows of this head's D columns
  __syncthreads();
  T* os = smem + wave * 32 * C::OST;
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4 vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = from_f32<T>(o[dt][4 * s + e] * inv);
      *(v4*)(os + lr * C::OST + dt * 32 + 8 * s + 4 * g) = vv;
    }
  if (!active) return;  // no further barrier: the stage of a wave is read by that wave only
  const int H = nh * D;
  constexpr int CPR = D / C::VE;       // vectors per output row
  constexpr int RPP = kWave / CPR;     // rows per pass
  T* out = ctx + ((size_t)b * Sq + qb * 32) * H + h * D;
#pragma unroll
  for (int p = 0; p < 32 / RPP; ++p) {
    const int row = p * RPP + lane / CPR, col = (lane % CPR) * C::VE;
    *(vec*)(out + (size_t)row * H + col) = *(const vec*)(os + row * C::OST + col);
  }
}

// 16-bit data: the same chain for up to 4 query blocks (128 queries) per workgroup, with Q,
// K and V^T going from global memory straight into LDS (buffer loads into LDS: no register
// staging, no LDS store instructions).  K and V^T stream through a ring of two chunk slots
// of up to 128 keys: chunk j + 1 is loading while chunk j is computed.  At 80 KB of LDS or
// less, two workgroups share a CU, so the loads, the stores and the matrix and vector phases
// of one overlap those of the other.
//
// Key order inside a 32-key tile: row i = 8a + 4h + b of the S^T tile (a < 4, h < 2, b < 4)
// is key attn_key(i) = 16h + 4a + b, so register r of lane (n, g) holds key 16g + r: a lane's
// 16 probabilities are 16 consecutive keys, and each P V^T fragment is 8 consecutive keys,
// one 16-byte LDS read of a V^T row.
__device__ __forceinline__ int attn_key(int i) {
  return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3);
}

// LDS rows are RB bytes of 16-byte chunks; chunk c of row r is stored at position
// c ^ swz(r).  A fragment read takes one chunk from each row of a group of lanes; the
// swizzles below give every pass of 8 lanes (128-byte bank window) or 16 lanes (256-byte
// window) distinct banks, for the rows those lanes read: rows lr for V^T and Q, rows
// attn_key(lr) for K.  They depend on r mod 32 only.
template <int RB> __device__ __forceinline__ int attn_swz_rows(int r) {
  if constexpr (RB == 256) return r & 15;
  else if constexpr (RB == 128) return (r & 7) ^ ((r >> 3) & 3);
  else return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}
template <int RB> __device__ __forceinline__ int attn_swz_keys(int r) {
  if constexpr (RB == 128) return (r & 7) ^ (((r >> 4) & 1) * 5);
  else return (r & 3) ^ ((r >> 2) & 1) ^ (((r >> 4) & 1) * 3);
}

template <typename T, int D, int SMAX, int CKMAX = 128> struct AttnDmaCfg {
  static constexpr int NW = SMAX / 32 < 4 ? SMAX / 32 : 4;  // waves (query blocks) per group
  static constexpr int CK = SMAX < CKMAX ? SMAX : CKMAX;    // keys per chunk
  static constexpr int NSLOT = SMAX / CK < 2 ? 1 : 2;       // ring slots
  static constexpr int CH = CK / 32;                        // key tiles per chunk
  static constexpr int KRB = D * 2;                         // bytes per K (and Q) row
  static constexpr int VRB = CK * 2;                        // bytes per V^T row of a chunk
  static constexpr int KBYTES = CK * KRB;                   // K of one chunk
  static constexpr int SLOT = KBYTES + D * VRB;             // K and V^T of one chunk
  static constexpr int QBYTES = NW * 32 * KRB;
  static constexpr int LDS = QBYTES + NSLOT * SLOT;
  static constexpr int KI = KBYTES / 1024;    // 1 KB load instructions per chunk of K
  static constexpr int VI = D * VRB / 1024;   // ... of V^T
  static constexpr int QI = 32 * KRB / 1024;  // ... per wave for its Q rows
  static constexpr int OST = D + 8;           // LDS row stride of the output stage (elements)
  static_assert(KI % NW == 0 && VI % NW == 0, "chunk loads split evenly over the waves");
  static_assert(LDS <= 80 * 1024, "two workgroups per CU");
  static constexpr int OCC = LDS <= 160 * 1024 / 3 ? 3 : 2;  // workgroups per CU by LDS
  static_assert(NW * 32 * OST * 2 <= LDS, "output stage must fit");
};

template <typename T, int D, int SMAX, int CKMAX = 128>
__global__ __launch_bounds__((AttnDmaCfg<T, D, SMAX, CKMAX>::NW * kWave),
                             (AttnDmaCfg<T, D, SMAX, CKMAX>::OCC)) void attention_dma_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ vt,
    const int32_t* __restrict__ lens, T* __restrict__ ctx, int B, int Sq, int Sk, int nh,
    float scale_log2e, int s_valid, int causal, int xcds) {
  typedef AttnDmaCfg<T, D, SMAX, CKMAX> C;
  typedef AttnMfma<T> MF;
  typedef typename MF::frag frag;
  typedef typename VecT<T, 4>::type v4;
  typedef typename Vec16<T>::type vec;
  static_assert(MF::VEC == 8, "16-bit data");
  constexpr int NQF = D / 16;   // 16-wide fragments along d
  constexpr int DT = D / 32;    // 32-row tiles of the transposed output along d
  constexpr int CH = C::CH;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  char* const Qs = smem;
  char* const ring = smem + C::QBYTES;   // slot z: K at ring + z SLOT, V^T after it

  const int qblocks = Sq / 32;
  const int groups = (qblocks + C::NW - 1) / C::NW;
  int blk = blockIdx.x;
  if (groups > 1 && xcds > 1 && (B * nh) % xcds == 0) {
    // workgroups go to the XCDs round-robin; renumber them so that the query groups of one
    // head run side by side on one XCD and its L2 serves the K/V^T reads after the first
    const int x = blk % xcds, slot = blk / xcds;
    blk = ((slot / groups) * xcds + x) * groups + slot % groups;
  }
  const int bh = blk / groups, grp = blk % groups;
  const int b = bh / nh, h = bh % nh;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 32, g = lane / 32;
  const int qb = grp * C::NW + wave;
  const bool active = qb < qblocks;
  int len = lens ? lens[b] : s_valid;
  len = min(max(len, 1), s_valid);
  int nkt = (len + 31) / 32;       // key tiles of this wave
  int nk = nkt * 32;               // keys the workgroup needs
  int clean = len / 32;            // leading key tiles that need no per-key mask
  if (causal) {
    // key tiles after a query block are entirely in its future
    nk = min(nkt, min(grp * C::NW + C::NW, qblocks)) * 32;
    nkt = min(nkt, qb + 1);
    clean = min(clean, qb);
  }
  const int query = qb * 32 + lr;
  const int nchunks = (nk + C::CK - 1) / C::CK;

  // Loads.  Lane l of a 1 KB load lands at position l % NC of LDS row (first row) + l / NC
  // and fetches the 16-byte chunk that belongs there.  The resources end at the head's last
  // K row / V^T element: rows or keys past Sk read as zero.
  constexpr int NCK = C::KRB / 16, NCV = C::VRB / 16;
  constexpr int KW = C::KI / C::NW, VW = C::VI / C::NW;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(k + (size_t)bh * Sk * D), (short)0, Sk * C::KRB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vt + (size_t)bh * D * Sk), (short)0, D * Sk * 2, 0x00020000);
  int koffg[KW], voffg[VW];
#pragma unroll
  for (int i = 0; i < KW; ++i) {
    const int r = (wave * KW + i) * (1024 / C::KRB) + lane / NCK;   // key within the chunk
    koffg[i] = r * C::KRB + (((lane % NCK) ^ attn_swz_keys<C::KRB>(r)) * 16);
  }
#pragma unroll
  for (int i = 0; i < VW; ++i) {
    const int r = (wave * VW + i) * (1024 / C::VRB) + lane / NCV;   // d
    voffg[i] = r * Sk * 2 + (((lane % NCV) ^ attn_swz_rows<C::VRB>(r)) * 16);
  }
  // chunk j into ring slot j % NSLOT: KW + VW loads of this wave
  auto load_chunk = [&](const int j, char* slot) {
#pragma unroll
    for (int i = 0; i < KW; ++i)
      lds_dma16(rk, koffg[i], slot + (wave * KW + i) * 1024, j * C::CK * C::KRB);
#pragma unroll
    for (int i = 0; i < VW; ++i)
      lds_dma16(rv, voffg[i], slot + C::KBYTES + (wave * VW + i) * 1024, j * C::CK * 2);
  };
  if (active) {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(q + ((size_t)bh * Sq + qb * 32) * D), (short)0, 32 * C::KRB, 0x00020000);
#pragma unroll
    for (int i = 0; i < C::QI; ++i) {
      const int r = i * (1024 / C::KRB) + lane / NCK;
      lds_dma16(rq, r * C::KRB + (((lane % NCK) ^ attn_swz_rows<C::KRB>(r)) * 16),
                Qs + wave * 32 * C::KRB + i * 1024);
    }
  }
  load_chunk(0, ring);

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float l_run = 1.f, m_run = -INFINITY;
  if (active) l_run = 0.f;

  // lane byte offsets of the fragment reads: chunk g + 2f of K row attn_key(lr) (of a tile)
  // and of Q row lr; chunk 4t + u + 2g of V^T row lr (of a 32-row d tile), keys
  // 32t + 16g + 8u .. + 7 of the chunk
  const int kr0 = attn_key(lr);
  int kq[NQF], vo[CH][2];
#pragma unroll
  for (int f = 0; f < NQF; ++f) kq[f] = kr0 * C::KRB + (((g + 2 * f) ^ attn_swz_keys<C::KRB>(kr0)) * 16);
#pragma unroll
  for (int t = 0; t < CH; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      vo[t][u] = lr * C::VRB + (((4 * t + u + 2 * g) ^ attn_swz_rows<C::VRB>(lr)) * 16);
  frag qf[NQF];

  // One chunk of CH key tiles from ring slot Z.  Chunks below `clean` run without a single
  // test; otherwise tiles past nkt are skipped (probabilities exactly 0) and keys are masked
  // key by key where a tile reaches len_b or the causal diagonal.
  auto chunk = [&](const int j, auto z, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    constexpr int Z = decltype(z)::value;
    const char* const kc = ring + Z * C::SLOT;
    const char* const vc = kc + C::KBYTES;
    const int c0 = j * CH;
    f32x16 sc[CH];
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      if (!TAIL || c0 + t < nkt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
#pragma unroll
        for (int f = 0; f < NQF; ++f)
          MF::mma(*(const frag*)(kc + t * 32 * C::KRB + kq[f]), qf[f], sc[t]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[t][r] = -INFINITY;
      }
    }
    if constexpr (TAIL) {
      // key of register r: tile*32 + 16*g + r
#pragma unroll
      for (int t = 0; t < CH; ++t) {
        const int kb = (c0 + t) * 32;
        if (c0 + t < nkt && (kb + 32 > len || (causal && kb + 31 > qb * 32))) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb + 16 * g + r;
            if (key >= len || (causal && key > query)) sc[t][r] = -INFINITY;
          }
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < CH; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
    // finite: every chunk's first key is below len and (causal) not after the query
    const float m_new = fmaxf(m_run, fmaxf(mx, half_swap(mx)));
    const float mc = m_new * scale_log2e;
    const float alpha = exp2_flush(fmaf(m_run, scale_log2e, -mc));  // 0 on the first chunk
    m_run = m_new;
    // probabilities in the storage type as the next MFMA's B operand: fragment u of a tile
    // holds registers 8u .. 8u+7, keys tile*32 + 16g + 8u .. + 7; the row sum adds exactly
    // these values
    frag pf[CH][2];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < CH; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[t][u][e] = from_f32<T>(exp2_flush(fmaf(sc[t][8 * u + e], scale_log2e, -mc)));
        psum = MF::sum(pf[t][u], psum);
      }
    l_run = l_run * alpha + (psum + half_swap(psum));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    // context: o[dt] += V^T[dt tile][keys] * P^T[keys][queries]; the V^T fragment of lane
    // (lr, g) for u is keys tile*32 + 16g + 8u .. + 7 of row 32 dt + lr, one 16-byte chunk
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      if (TAIL && c0 + t >= nkt) continue;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          MF::mma(*(const frag*)(vc + dt * 32 * C::VRB + vo[t][u]), pf[t][u], o[dt]);
    }
  };
  // Chunk j: wait for its loads (the only ones in flight), a barrier that publishes them and
  // that every wave passes only after finishing chunk j - 1, then the loads of chunk j + 1
  // into the slot chunk j - 1 used, then the chunk itself.
  auto step = [&](const int j, auto z) {
    constexpr int Z = decltype(z)::value;
    wait_vmcnt<0>();
    workgroup_barrier();
    if (j + 1 < nchunks) load_chunk(j + 1, ring + ((Z + 1) % C::NSLOT) * C::SLOT);
    if (!active) return;
    if (j == 0) {
      const char* qs = Qs + wave * 32 * C::KRB;
#pragma unroll
      for (int f = 0; f < NQF; ++f)
        qf[f] = *(const frag*)(qs + lr * C::KRB + (((g + 2 * f) ^ attn_swz_rows<C::KRB>(lr)) * 16));
    }
    if ((j + 1) * CH <= clean) chunk(j, z, std::false_type{});
    else if (j * CH < nkt) chunk(j, z, std::true_type{});
  };
  for (int j = 0; j < nchunks; j += C::NSLOT) {
    step(j, std::integral_constant<int, 0>{});
    if constexpr (C::NSLOT == 2)
      if (j + 1 < nchunks) step(j + 1, std::integral_constant<int, 1>{});
  }

  // normalise, stage [query][d] in LDS (free once every wave is past its last chunk), then
  // store whole rows of this head's D columns
  __syncthreads();
  T* os = (T*)smem + wave * 32 * C::OST;
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      v4 vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = from_f32<T>(o[dt][4 * s4 + e] * inv);
      *(v4*)(os + lr * C::OST + dt * 32 + 8 * s4 + 4 * g) = vv;
    }
  if (!active) return;  // no further barrier: the stage of a wave is read by that wave only
  const int H = nh * D;
  constexpr int VE = 8;                // elements per 16-byte vector
  constexpr int CPR = D / VE;          // vectors per output row
  constexpr int RPP = kWave / CPR;     // rows per pass
  T* out = ctx + ((size_t)b * Sq + qb * 32) * H + h * D;
#pragma unroll
  for (int p = 0; p < 32 / RPP; ++p) {
    const int row = p * RPP + lane / CPR, col = (lane % CPR) * VE;
    *(vec*)(out + (size_t)row * H + col) = *(const vec*)(os + row * C::OST + col);
  }
}

// S <= 32 (one 32-key tile per head), 16-bit data: the same chain with every MFMA operand
// read straight from global memory in fragment layout -- Q and K rows as 16-byte loads, V^T
// as two 8-byte loads per fragment -- and the output stored from registers as 8-byte runs
// of four consecutive d, so a wave needs no LDS and no barrier and all of its loads are in
// flight at once.  One wave per (sequence, head), four per workgroup.
template <typename T, int D>
__global__ __launch_bounds__(256) void attention_s32_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ k,
                                                           const T* __restrict__ vt,
                                                           const int32_t* __restrict__ lens,
                                                           T* __restrict__ ctx, int B, int S,
                                                           int nh, float scale_log2e,
                                                           int s_valid, int causal) {
  typedef AttnMfma<T> MF;
  typedef typename MF::frag frag;
  typedef typename VecT<T, 4>::type v4;
  constexpr int VEC = MF::VEC;
  static_assert(VEC == 8, "16-bit data");
  constexpr int KF = 2 * VEC;  // d consumed per fragment pair
  constexpr int NQF = D / KF;
  constexpr int DT = D / 32;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int bh = blockIdx.x * (blockDim.x / kWave) + wave;
  if (bh >= B * nh) return;  // whole waves leave; no barrier follows
  const int b = bh / nh, h = bh % nh;
  const int lr = lane % 32, g = lane / 32;
  int len = lens ? lens[b] : s_valid;
  len = min(max(len, 1), s_valid);

  // query lr of Q, key lr of K (rows past S are never read: S is 32 here)
  frag qf[NQF], kf[NQF];
  const T* qp = q + ((size_t)bh * S + lr) * D + g * VEC;
  const T* kp = k + ((size_t)bh * S + lr) * D + g * VEC;
#pragma unroll
  for (int f = 0; f < NQF; ++f) {
    qf[f] = *(const frag*)(qp + f * KF);
    kf[f] = *(const frag*)(kp + f * KF);
  }
  // V^T rows d = dt*32 + lr, keys 16u + 4g + {0..3} and {8..11}
  frag vf[DT][2];
  const T* vp = vt + ((size_t)bh * D + lr) * S + 4 * g;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const v4 lo = *(const v4*)(vp + (size_t)dt * 32 * S + 16 * u);
      const v4 hi = *(const v4*)(vp + (size_t)dt * 32 * S + 16 * u + 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[dt][u][e] = lo[e];
        vf[dt][u][e + 4] = hi[e];
      }
    }

  // S^T = K Q^T: register r of a lane holds key 8(r/4) + 4g + r%4 of query lr
  f32x16 sc;
#pragma unroll
  for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
  for (int f = 0; f < NQF; ++f) MF::mma(kf[f], qf[f], sc);
  float mx = -INFINITY;
  if (len < 32 || causal) {  // the per-key mask, only when some key is masked
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r / 4) + 4 * g + (r % 4);
      if (key >= len || (causal && key > lr)) sc[r] = -INFINITY;
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));  // finite: key 0 is always valid
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sc[r] = exp2_flush((sc[r] - mx) * scale_log2e);
    sum += sc[r];
  }
  sum += __shfl_xor(sum, 32);

  // C^T = V^T P^T; MFMA u consumes P registers 8u..8u+7 = keys 16u + {0..3, 8..11} + 4g
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    frag pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = from_f32<T>(sc[8 * u + e]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) MF::mma(vf[dt][u], pf, o[dt]);
  }

  // register r of o[dt]: d = dt*32 + 8(r/4) + 4g + r%4 of query lr
  const float inv = 1.0f / sum;
  T* out = ctx + ((size_t)b * S + lr) * (nh * D) + h * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      v4 vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = from_f32<T>(o[dt][4 * s4 + e] * inv);
      *(v4*)(out + dt * 32 + 8 * s4) = vv;
    }
}

// The S = 32 attention of one (sequence, head) followed by that head's share of the
// attention-output projection, for small batches where that projection splits K and the
// LayerNorm after it sums the split partials: the projection's K range is the merged-heads
// dimension, so head h's slice of it is exactly C_h (the head's context, 32 x D) times rows
// h*D .. h*D+D-1 of Wo.  ceil(H / 256) workgroups of 8 waves per (b, h), one 32-column
// output tile per wave (tile j = 8 part + wave): every wave first issues the loads of its Wo
// fragments (the weight is given transposed, wo_t[n][k], so a fragment row is 4 consecutive
// k twice; wave 0 after its Q, K, V loads), wave 0 runs
// attention_s32_kernel's chain and leaves C_h, rounded to the storage type as the context
// would be stored, in LDS in its own register order; after one barrier each wave multiplies
// its tiles, C_h fragments taken lane by lane in that register order (the K order of an
// MFMA only has to agree between its operands, and the Wo fragments are loaded in the same
// order), and stores the fp32 partial tile to p[h][b*32 + i][n].  One launch for what the
// attention kernel and the split-K partial products of the projection did in two.
constexpr int kAttnOutMaxHidden = 1024;

template <typename T, int D>
__global__ __launch_bounds__(512) void attention_oproj_s32_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ vt,
    const int32_t* __restrict__ lens, const T* __restrict__ wo_t, float* __restrict__ p, int B,
    int nh, float scale_log2e, int s_valid) {
  typedef AttnMfma<T> MF;
  typedef typename MF::frag frag;
  typedef typename VecT<T, 4>::type v4;
  constexpr int VEC = MF::VEC;
  static_assert(VEC == 8, "16-bit data");
  constexpr int S = 32, KF = 2 * VEC, NQF = D / KF, DT = D / 32;
  constexpr int NST = D / 16;  // MFMA K steps over the head's D columns
  __shared__ __attribute__((aligned(16))) T cs[kWave * 16 * DT];  // C_h, lane by lane
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lr = lane % 32, g = lane / 32;
  const int H = nh * D, ntiles = H / 32, parts = (ntiles + 7) / 8;
  const int bh = blockIdx.x / parts, part = blockIdx.x % parts, b = bh / nh, h = bh % nh;
  const int j = 8 * part + wave;  // this wave's output column tile

  // step st of an MFMA over the head's columns takes register pairs 2 st and 2 st + 1 of a
  // lane (pair i: dt = i / 4, q = i % 4, i.e. d = 32 dt + 8 q + 4 g + 0..3)
  frag wf[NST];
  auto load_wo = [&]() {
    if (j < ntiles) {
      const T* wr = wo_t + (size_t)(32 * j + lr) * H + h * D + 4 * g;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int i0 = 2 * st, i1 = 2 * st + 1;
        const v4 lo = *(const v4*)(wr + 32 * (i0 / 4) + 8 * (i0 % 4));
        const v4 hi = *(const v4*)(wr + 32 * (i1 / 4) + 8 * (i1 % 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wf[st][e] = lo[e];
          wf[st][e + 4] = hi[e];
        }
      }
    }
  };
  if (wave != 0) load_wo();

  if (wave == 0) {
    int len = lens ? lens[b] : s_valid;
    len = min(max(len, 1), s_valid);
    frag qf[NQF], kf[NQF];
    const T* qp = q + ((size_t)bh * S + lr) * D + g * VEC;
    const T* kp = k + ((size_t)bh * S + lr) * D + g * VEC;
#pragma unroll
    for (int f = 0; f < NQF; ++f) {
      qf[f] = *(const frag*)(qp + f * KF);
      kf[f] = *(const frag*)(kp + f * KF);
    }
    frag vf[DT][2];
    const T* vp = vt + ((size_t)bh * D + lr) * S + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const v4 lo = *(const v4*)(vp + (size_t)dt * 32 * S + 16 * u);
        const v4 hi = *(const v4*)(vp + (size_t)dt * 32 * S + 16 * u + 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[dt][u][e] = lo[e];
          vf[dt][u][e + 4] = hi[e];
        }
      }
    load_wo();
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int f = 0; f < NQF; ++f) MF::mma(kf[f], qf[f], sc);
    float mx = -INFINITY;
    if (len < 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r / 4) + 4 * g + (r % 4);
        if (key >= len) sc[r] = -INFINITY;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));  // finite: key 0 is always valid
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = exp2_flush((sc[r] - mx) * scale_log2e);
      sum += sc[r];
    }
    sum += __shfl_xor(sum, 32);
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      frag pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = from_f32<T>(sc[8 * u + e]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) MF::mma(vf[dt][u], pf, o[dt]);
    }
    // register r of o[dt]: d = 32 dt + 8 (r / 4) + 4 g + r % 4 of query lr; pair i = 4 dt + r / 4
    const float inv = 1.0f / sum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) cs[(16 * dt + r) * kWave + lane] = from_f32<T>(o[dt][r] * inv);
  }
  __syncthreads();
  // C_h fragment of step st for lane (query lr, g): pairs 2 st, 2 st + 1 of that lane
  frag cf[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int e = 0; e < 8; ++e) cf[st][e] = cs[(8 * st + e) * kWave + lane];
  // partial tile j: register r of a lane is column 32 j + 8 (r / 4) + 4 g + r % 4 of query lr
  if (j >= ntiles) return;
  float* pr = p + ((size_t)h * B * S + (size_t)b * S + lr) * H;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int st = 0; st < NST; ++st) MF::mma(wf[st], cf[st], acc);
#pragma unroll
  for (int qq = 0; qq < 4; ++qq)
    *(f32x4*)(pr + 32 * j + 8 * qq + 4 * g) =
        f32x4{acc[4 * qq], acc[4 * qq + 1], acc[4 * qq + 2], acc[4 * qq + 3]};
}

bool attention_out_partials_fit(ftx_dtype dt, int S, int nh, int d) {
  return dt != FTX_FP32 && S == 32 && (d == 32 || d == 64) && nh * d % 32 == 0 &&
         nh * d <= kAttnOutMaxHidden;
}

hipError_t launch_attention_out_partials(ftx_dtype dt, int B, int nh, int d, const void* q,
                                         const void* k, const void* vt, const int32_t* lens,
                                         int s_valid, const void* wo_t, float* p, hipStream_t s) {
  if (!attention_out_partials_fit(dt, 32, nh, d) || B < 1) return hipErrorInvalidValue;
  if (s_valid <= 0 || s_valid > 32) s_valid = 32;
  const float scale_log2e = (float)(1.4426950408889634 / sqrt((double)d));
  const unsigned grid = (unsigned)(B * nh * ((nh * d / 32 + 7) / 8));
#define FTX_AOP(T, D)                                                                            \
  attention_oproj_s32_kernel<T, D><<<grid, 512, 0, s>>>((const T*)q, (const T*)k, (const T*)vt,  \
                                                        lens, (const T*)wo_t, p, B, nh,         \
                                                        scale_log2e, s_valid)
  if (dt == FTX_FP16) {
    if (d == 64) FTX_AOP(f16, 64); else FTX_AOP(f16, 32);
  } else {
    if (d == 64) FTX_AOP(bf16, 64); else FTX_AOP(bf16, 32);
  }
#undef FTX_AOP
  return hipGetLastError();
}

constexpr size_t kMaxLdsBytes = 160 * 1024;  // per workgroup on gfx950

template <typename T, int D, int SMAX>
static hipError_t attn_launch_cfg(int B, int Sq, int Sk, int nh, const void* q, const void* k,
                                  const void* vt, const int32_t* lens, void* ctx,
                                  float scale_log2e, int s_valid, int causal, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    typedef AttnDmaCfg<T, D, SMAX> C;
    const int groups = (Sq / 32 + C::NW - 1) / C::NW;
    attention_dma_kernel<T, D, SMAX><<<B * nh * groups, C::NW * kWave, 0, s>>>(
        (const T*)q, (const T*)k, (const T*)vt, lens, (T*)ctx, B, Sq, Sk, nh, scale_log2e,
        s_valid, causal, device_info().xcds);
  } else {
    typedef AttnCfg<T, D, SMAX> C;
    const int groups = (Sq / 32 + C::NW - 1) / C::NW;
    attention_kernel<T, D, SMAX><<<B * nh * groups, C::NW * kWave, 0, s>>>(
        (const T*)q, (const T*)k, (const T*)vt, lens, (T*)ctx, B, Sq, Sk, nh, scale_log2e,
        s_valid, causal, device_info().xcds);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t attn_launch_d(int B, int Sq, int Sk, int nh, const void* q, const void* k,
                                const void* vt, const int32_t* lens, void* ctx,
                                float scale_log2e, int s_valid, int causal, hipStream_t s) {
  if (Sk <= 32) {
    // the register-only kernel has the shorter chain (no LDS round trip, no barrier) and wins
    // while few heads are in flight; with thousands its 32-row fragment loads cost more in
    // address processing than the LDS kernel's contiguous 1 KB staging loads (measured at
    // BERT-base: 6.9 vs 8.8 us at 768 heads, 25.9 vs 23.5 us at 6144)
    if constexpr (sizeof(T) == 2) if (Sq == 32 && B * nh <= 2048) {
      attention_s32_kernel<T, D><<<(B * nh + 3) / 4, 256, 0, s>>>(
          (const T*)q, (const T*)k, (const T*)vt, lens, (T*)ctx, B, 32, nh, scale_log2e, s_valid,
          causal);
      return hipGetLastError();
    }
    return attn_launch_cfg<T, D, 32>(B, Sq, Sk, nh, q, k, vt, lens, ctx, scale_log2e, s_valid, causal, s);
  }
  if (Sk <= 64) return attn_launch_cfg<T, D, 64>(B, Sq, Sk, nh, q, k, vt, lens, ctx, scale_log2e, s_valid, causal, s);
  if (Sk <= 128) return attn_launch_cfg<T, D, 128>(B, Sq, Sk, nh, q, k, vt, lens, ctx, scale_log2e, s_valid, causal, s);
  if (Sk <= 256) return attn_launch_cfg<T, D, 256>(B, Sq, Sk, nh, q, k, vt, lens, ctx, scale_log2e, s_valid, causal, s);
  if constexpr (AttnCfg<T, D, 512>::LDS * sizeof(T) <= kMaxLdsBytes)
    return attn_launch_cfg<T, D, 512>(B, Sq, Sk, nh, q, k, vt, lens, ctx, scale_log2e, s_valid, causal, s);
  const int blocks = (B * nh * (Sq / 32) + 3) / 4;
  attention_global_kernel<T, D><<<blocks, 256, 0, s>>>((const T*)q, (const T*)k, (const T*)vt, lens,
                                                       (T*)ctx, B, Sq, Sk, nh, scale_log2e, s_valid,
                                                       causal);
  return hipGetLastError();
}

template <typename T>
static hipError_t attn_launch(int B, int Sq, int Sk, int nh, int d, const void* q, const void* k,
                              const void* vt, const int32_t* lens, void* ctx, hipStream_t s,
                              int s_valid, int causal) {
  const float scale_log2e = (float)(1.4426950408889634 / sqrt((double)d));
  if (d == 64) return attn_launch_d<T, 64>(B, Sq, Sk, nh, q, k, vt, lens, ctx, scale_log2e, s_valid, causal, s);
  if (d == 32) return attn_launch_d<T, 32>(B, Sq, Sk, nh, q, k, vt, lens, ctx, scale_log2e, s_valid, causal, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attention(ftx_dtype dt, int B, int Sq, int Sk, int nh, int d, const void* q,
                            const void* k, const void* vt, const int32_t* lens, void* ctx,
                            hipStream_t s, int s_valid, bool causal) {
  if (s_valid <= 0 || s_valid > Sk) s_valid = Sk;
  const int c = causal ? 1 : 0;
  switch (dt) {
    case FTX_FP32: return attn_launch<float>(B, Sq, Sk, nh, d, q, k, vt, lens, ctx, s, s_valid, c);
    case FTX_FP16: return attn_launch<f16>(B, Sq, Sk, nh, d, q, k, vt, lens, ctx, s, s_valid, c);
    case FTX_BF16: return attn_launch<bf16>(B, Sq, Sk, nh, d, q, k, vt, lens, ctx, s, s_valid, c);
  }
  return hipErrorInvalidValue;
}

}  // namespace ftx
