// Device kernels of the self-speculative decoding engine, written for gfx950
// (CDNA4: wave64, MFMA, 160 KB LDS per CU).
//
// Every kernel computes each output row from that row's inputs only, with a
// reduction order that depends on the problem size (K, key positions) but
// never on the number of rows in the launch.  A verify row therefore gets
// bit-identical results to the autoregressive step at the same position,
// which is what makes greedy self-speculative decoding lossless on the GPU
// itself (CLaSp article, section 3: the full model's prediction is final).
// No floating-point atomics are used anywhere.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lss {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
template <typename T> __device__ __forceinline__ float ld_elem(const T* p, size_t i);
template <> __device__ __forceinline__ float ld_elem<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p, size_t i) { return bf2f(p[i]); }
template <typename T> __device__ __forceinline__ void st_elem(T* p, size_t i, float v);
template <> __device__ __forceinline__ void st_elem<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st_elem<uint16_t>(uint16_t* p, size_t i, float v) { p[i] = f2bf(v); }

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// Block-wide sum in a fixed order (wave tree, then waves in index order).
// `red` holds >= blockDim/64 floats; returns the total to every thread.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = red[0];
  for (int i = 1; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

// ---------------------------------------------------------------- small kernels
__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

// h[m][:] = E[tok[m]][:]  (float32 residual stream)
template <typename WT>
__global__ void k_embed(const WT* __restrict__ E, const int32_t* __restrict__ tok, int d,
                        float* __restrict__ h, int ldh) {
  const int m = blockIdx.x;
  const size_t row = (size_t)tok[m] * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) h[(size_t)m * ldh + i] = ld_elem<WT>(E, row + i);
}

// Symmetric per-token int8 codes of n values held by this thread group.
// inv = fl32(127 / amax) (correctly rounded), q = clamp(rint(x * inv), +-127).
__device__ __forceinline__ float quant_code(float x, float inv) {
  float q = rintf(__fmul_rn(x, inv));
  return fminf(fmaxf(q, -127.f), 127.f);
}

#define LSS_NORM_THREADS 256
#define LSS_NORM_PER_THREAD 32   // d_model <= 8192

// RMSNorm of rows of h: x = h / sqrt(mean(h^2) + eps) * g, optionally
// followed by int8 quantization (x replaced by its integer codes, xs[m] =
// amax/127).  Without quantization xs[m] = 1.
template <typename GT>
__global__ __launch_bounds__(LSS_NORM_THREADS) void k_rmsnorm(const float* __restrict__ h, int ldh,
                                                              const GT* __restrict__ g, int d, float eps,
                                                              float* __restrict__ x, int ldx,
                                                              float* __restrict__ xs, int quant) {
  __shared__ float red[LSS_NORM_THREADS / 64];
  const int m = blockIdx.x;
  const float* hr = h + (size_t)m * ldh;
  float v[LSS_NORM_PER_THREAD];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < LSS_NORM_PER_THREAD; ++j) {
    const int i = threadIdx.x + j * LSS_NORM_THREADS;
    v[j] = (i < d) ? hr[i] : 0.f;
    ss = __fadd_rn(ss, __fmul_rn(v[j], v[j]));
  }
  ss = block_sum(ss, red);
  const float rstd = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(ss, (float)d), eps)));
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < LSS_NORM_PER_THREAD; ++j) {
    const int i = threadIdx.x + j * LSS_NORM_THREADS;
    if (i < d) v[j] = __fmul_rn(__fmul_rn(v[j], rstd), ld_elem<GT>(g, i));
    amax = fmaxf(amax, fabsf(v[j]));
  }
  float* xr = x + (size_t)m * ldx;
  if (!quant) {
#pragma unroll
    for (int j = 0; j < LSS_NORM_PER_THREAD; ++j) {
      const int i = threadIdx.x + j * LSS_NORM_THREADS;
      if (i < d) xr[i] = v[j];
    }
    if (threadIdx.x == 0) xs[m] = 1.0f;
    return;
  }
  amax = block_max(amax, red);
  const float inv = amax > 0.f ? __fdiv_rn(127.0f, amax) : 0.f;
#pragma unroll
  for (int j = 0; j < LSS_NORM_PER_THREAD; ++j) {
    const int i = threadIdx.x + j * LSS_NORM_THREADS;
    if (i < d) xr[i] = quant_code(v[j], inv);
  }
  if (threadIdx.x == 0) xs[m] = __fdiv_rn(amax, 127.0f);
}

// In-place int8 quantization of rows x[m][0..n) (codes as float, or into q8),
// scale -> xs[m].  Used for the attention output and the SwiGLU output of a
// quantized draft layer, and by the stand-alone quantization entry point.
__global__ __launch_bounds__(256) void k_quant_rows(float* __restrict__ x, int ldx, int n,
                                                   float* __restrict__ xs, int8_t* __restrict__ q8) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  float* xr = x + (size_t)m * ldx;
  float amax = 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) amax = fmaxf(amax, fabsf(xr[i]));
  amax = block_max(amax, red);
  const float inv = amax > 0.f ? __fdiv_rn(127.0f, amax) : 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const float q = quant_code(xr[i], inv);
    if (q8) q8[(size_t)m * n + i] = (int8_t)q;
    else xr[i] = q;
  }
  if (threadIdx.x == 0) xs[m] = __fdiv_rn(amax, 127.0f);
}

// ---------------------------------------------------------------- small-M MFMA GEMM
// Y[m][n] = sum_k X[m][k] * W[n][k] for m < M <= 16*MT, weights row-major
// [N][K] streamed once from HBM.  One workgroup = one 16-column tile of N and
// GEMM_WAVES waves that split K into fixed contiguous ranges; the waves'
// partial tiles are summed in LDS in wave order.  The K split, the per-lane
// k assignment and the MFMA sequence depend only on K, so row m's result is
// the same for every M (rows are independent MFMA rows; padding rows are 0).
//
// MFMA operand use (16x16x32 bf16 / 16x16x4 f32): lane l supplies A row
// (l & 15) = activation row, B column (l & 15) = weight row, over a k group
// chosen by (l >> 4).  Because a dot product does not depend on which k a
// lane holds as long as A and B agree, each lane reads 4 consecutive 16-byte
// vectors of its weight row (64 contiguous bytes; 256 bytes per row per
// wave step), the activation values at the same k, and feeds them to 4 (bf16)
// or 16 (f32) MFMAs.  bf16 weights: the float32 activation is split into
// hi = bf16(x) and lo = bf16(x - hi) and both are multiplied (two MFMAs), so
// the activation keeps ~16 significant bits; int8 codes are exact in hi.
#define GEMM_WAVES 8
#define GEMM_U 4

enum { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

struct GemmArgs {
  const void* w[3];      // weight segments stacked along N
  int nseg[3];           // rows per segment (multiples of 16)
  const void* w2;        // SWIGLU: up-projection weights [N][K]
  int N, K;
  const float* X; int ldx; int M;
  const float* xs;       // per-row scale of X (int8 codes) or nullptr
  float* Y; int ldy;
  const float* R; int ldr;  // RESID: residual input
  float* part;           // LOGITS: per (row, tile) {max, argmax bits, sum exp}
};

template <typename WT> struct WTr;
template <> struct WTr<uint16_t> { static constexpr int EPL = 8; };  // bf16: 8 per 16 bytes
template <> struct WTr<float> { static constexpr int EPL = 4; };

__device__ __forceinline__ void split_bf16(const float* v, bf16x8_t& hi, bf16x8_t& lo) {
  u16x8 h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t hb = f2bf(v[e]);
    h[e] = hb;
    l[e] = f2bf(__fsub_rn(v[e], bf2f(hb)));
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  lo = __builtin_bit_cast(bf16x8_t, l);
}

template <typename WT, int MT>
__device__ __forceinline__ void gemm_step(const uint4 (&w)[GEMM_U], const float (&a)[MT][GEMM_U][WTr<WT>::EPL],
                                          f32x4 (&acc)[MT]) {
  if constexpr (sizeof(WT) == 2) {
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u) {
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, w[u]);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        bf16x8_t hi, lo;
        split_bf16(a[t][u], hi, lo);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc[t], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u) {
      const float wf[4] = {__uint_as_float(w[u].x), __uint_as_float(w[u].y), __uint_as_float(w[u].z),
                           __uint_as_float(w[u].w)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t][u][e], wf[e], acc[t], 0, 0, 0);
    }
  }
}

template <typename WT>
__device__ __forceinline__ void load_w(uint4 (&w)[GEMM_U], const WT* row, int kb, int K, bool ok) {
  constexpr int EPL = WTr<WT>::EPL;
#pragma unroll
  for (int u = 0; u < GEMM_U; ++u) {
    const int k = kb + u * EPL;
    if (ok && k < K) w[u] = *reinterpret_cast<const uint4*>(row + k);
    else w[u] = make_uint4(0, 0, 0, 0);
  }
}

template <typename WT, int MT>
__device__ __forceinline__ void load_a(float (&a)[MT][GEMM_U][WTr<WT>::EPL], const float* X, int ldx, int M,
                                       int r, int kb, int K) {
  constexpr int EPL = WTr<WT>::EPL;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = t * 16 + r;
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u) {
      const int k = kb + u * EPL;
      if (m < M && k < K) {
        const float4* p = reinterpret_cast<const float4*>(X + (size_t)m * ldx + k);
#pragma unroll
        for (int e4 = 0; e4 < EPL / 4; ++e4) {
          const float4 f = p[e4];
          a[t][u][e4 * 4 + 0] = f.x; a[t][u][e4 * 4 + 1] = f.y;
          a[t][u][e4 * 4 + 2] = f.z; a[t][u][e4 * 4 + 3] = f.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) a[t][u][e] = 0.f;
      }
    }
  }
}

// ONE = the launch has exactly one row (draft steps, greedy steps): the same
// arithmetic as MT = 1, compiled separately so profiles attribute it apart.
template <typename WT, int MT, int EPI, bool ONE>
__global__ __launch_bounds__(64 * GEMM_WAVES) void k_gemm(GemmArgs ga) {
  constexpr int EPL = WTr<WT>::EPL;
  constexpr int KS = 4 * EPL * GEMM_U;  // k per wave step
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  __shared__ float red[NACC][MT][GEMM_WAVES][64][4];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  // weight segment of this tile
  int seg = 0, nloc = n0;
  while (seg < 2 && nloc >= ga.nseg[seg]) { nloc -= ga.nseg[seg]; ++seg; }
  const bool row_ok = (n0 + r) < ga.N;
  const WT* wrow = reinterpret_cast<const WT*>(ga.w[seg]) + (size_t)(row_ok ? nloc + r : 0) * ga.K;
  const WT* wrow2 = (EPI == EPI_SWIGLU)
                        ? reinterpret_cast<const WT*>(ga.w2) + (size_t)(row_ok ? n0 + r : 0) * ga.K
                        : nullptr;
  const int K = ga.K;
  const int nsteps = (K + KS - 1) / KS;
  const int s0 = (wave * nsteps) / GEMM_WAVES, s1 = ((wave + 1) * nsteps) / GEMM_WAVES;

  f32x4 acc[NACC][MT];
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (s0 < s1) {
    uint4 wc[NACC][GEMM_U], wn[NACC][GEMM_U];
    float ac[MT][GEMM_U][EPL];
    int kb = s0 * KS + g * EPL * GEMM_U;
    load_w<WT>(wc[0], wrow, kb, K, row_ok);
    if constexpr (NACC == 2) load_w<WT>(wc[1], wrow2, kb, K, row_ok);
    for (int s = s0; s < s1; ++s) {
      load_a<WT, MT>(ac, ga.X, ga.ldx, ONE ? 1 : ga.M, r, kb, K);
      const int kn = kb + KS;
      if (s + 1 < s1) {
        load_w<WT>(wn[0], wrow, kn, K, row_ok);
        if constexpr (NACC == 2) load_w<WT>(wn[1], wrow2, kn, K, row_ok);
      }
      gemm_step<WT, MT>(wc[0], ac, acc[0]);
      if constexpr (NACC == 2) gemm_step<WT, MT>(wc[1], ac, acc[1]);
#pragma unroll
      for (int q = 0; q < NACC; ++q)
#pragma unroll
        for (int u = 0; u < GEMM_U; ++u) wc[q][u] = wn[q][u];
      kb = kn;
    }
  }
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[q][t][wave][lane][j] = acc[q][t][j];
  __syncthreads();
  if (wave >= MT) return;
  const int t = wave;
  float v[NACC][4];
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = red[q][t][0][lane][j];
#pragma unroll
      for (int w = 1; w < GEMM_WAVES; ++w) s = __fadd_rn(s, red[q][t][w][lane][j]);
      v[q][j] = s;
    }
  // lane (r, g) holds D[row 16t + 4g + j][column n0 + r]
  const int n = n0 + r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = t * 16 + 4 * g + j;
    const bool ok = (m < ga.M) && (n < ga.N);
    float y = v[0][j];
    if (ga.xs && m < ga.M) y = __fmul_rn(y, ga.xs[m]);
    if constexpr (EPI == EPI_STORE) {
      if (ok) ga.Y[(size_t)m * ga.ldy + n] = y;
    } else if constexpr (EPI == EPI_RESID) {
      if (ok) ga.Y[(size_t)m * ga.ldy + n] = __fadd_rn(ga.R[(size_t)m * ga.ldr + n], y);
    } else if constexpr (EPI == EPI_SWIGLU) {
      float u = v[1][j];
      if (ga.xs && m < ga.M) u = __fmul_rn(u, ga.xs[m]);
      const float sg = __fdiv_rn(y, __fadd_rn(1.0f, expf(-y)));
      if (ok) ga.Y[(size_t)m * ga.ldy + n] = __fmul_rn(sg, u);
    } else {  // EPI_LOGITS: store and reduce the 16 columns of row m held by lanes 16g..16g+15
      if (ok) ga.Y[(size_t)m * ga.ldy + n] = y;
      float mx = (n < ga.N) ? y : -INFINITY;
      int idx = n;
      for (int o = 8; o >= 1; o >>= 1) {
        const float om = __shfl_xor(mx, o, 16);
        const int oi = __shfl_xor(idx, o, 16);
        if (om > mx || (om == mx && oi < idx)) { mx = om; idx = oi; }
      }
      float e = (n < ga.N) ? expf(__fsub_rn(y, mx)) : 0.f;
      // fixed-order sum over the 16 lanes
      for (int o = 8; o >= 1; o >>= 1) e = __fadd_rn(e, __shfl_xor(e, o, 16));
      if (r == 0 && m < ga.M) {
        float* p = ga.part + ((size_t)m * gridDim.x + blockIdx.x) * 3;
        p[0] = mx;
        p[1] = __int_as_float(idx);
        p[2] = e;
      }
    }
  }
}

// ---------------------------------------------------------------- RoPE + KV append
// qkv[m] = [q (Hq*hd) | k (Hkv*hd) | v (Hkv*hd)] from the fused projection.
// Rotates q and k by the rotate-half rule at position pos0 + m*pos_step with
// the host-built cos/sin table, writes q to qrot and k, v either into the
// layer's KV cache ([Hkv][max_seq][hd]) or, for layer-selection rows, into
// selfkv[m][2][Hkv][hd] (those rows' own key/value, never cached).
template <typename KT>
__global__ void k_rope_kv(const float* __restrict__ qkv, int ldqkv, int Hq, int Hkv, int hd,
                          const float2* __restrict__ cs, int pos0, int pos_step, float* __restrict__ qrot,
                          KT* __restrict__ kc, KT* __restrict__ vc, int max_seq, float* __restrict__ selfkv) {
  const int m = blockIdx.x, h = blockIdx.y;
  const int half = hd / 2;
  const int pos = pos0 + m * pos_step;
  const float* src = qkv + (size_t)m * ldqkv + (size_t)h * hd;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const float x1 = src[i], x2 = src[i + half];
    if (h < Hq + Hkv) {
      const float2 c = cs[(size_t)pos * half + i];
      const float y1 = __fsub_rn(__fmul_rn(x1, c.x), __fmul_rn(x2, c.y));
      const float y2 = __fadd_rn(__fmul_rn(x2, c.x), __fmul_rn(x1, c.y));
      if (h < Hq) {
        float* q = qrot + ((size_t)m * Hq + h) * hd;
        q[i] = y1;
        q[i + half] = y2;
      } else {
        const int kh = h - Hq;
        if (selfkv) {
          float* k = selfkv + (((size_t)m * 2 + 0) * Hkv + kh) * hd;
          k[i] = y1;
          k[i + half] = y2;
        } else {
          const size_t o = ((size_t)kh * max_seq + pos) * hd;
          st_elem<KT>(kc, o + i, y1);
          st_elem<KT>(kc, o + i + half, y2);
        }
      }
    } else {
      const int kh = h - Hq - Hkv;
      if (selfkv) {
        float* v = selfkv + (((size_t)m * 2 + 1) * Hkv + kh) * hd;
        v[i] = x1;
        v[i + half] = x2;
      } else {
        const size_t o = ((size_t)kh * max_seq + pos) * hd;
        st_elem<KT>(vc, o + i, x1);
        st_elem<KT>(vc, o + i + half, x2);
      }
    }
  }
}

// ---------------------------------------------------------------- attention
// Split-key attention.  Keys are cut into fixed 64-position chunks of the
// cache (absolute positions), so a row's chunks do not depend on the other
// rows of the launch.  Row m sees cache position u iff
//   u < lim_base + m*lim_step            (committed prefix / causal rows)
//   or u - wbase in [0, 32) with bit (u - wbase) of wmask set
//                                       (draft window slots this layer wrote)
// plus, for layer-selection rows, its own key/value (added by the combine).
#define ATT_CH 64
#define ATT_QB 32
#define ATT_THREADS 256

struct AttnArgs {
  const void* kc; const void* vc;  // layer cache [Hkv][max_seq][hd]
  int max_seq, Hq, Hkv, hd, M;
  const float* qrot;               // [M][Hq][hd]
  int lim_base, lim_step, wbase;
  uint32_t wmask;
  int nch;                         // chunks in this launch
  float* part;                     // [M][Hq][nch_max][hd + 2]
  int nch_max;
  float scale;                     // 1/sqrt(hd)
};

template <typename KT, int HD>
__global__ __launch_bounds__(ATT_THREADS) void k_attn_partial(AttnArgs a) {
  __shared__ float kv_s[ATT_CH][HD + 1];
  __shared__ float q_s[ATT_QB][HD];
  __shared__ float p_s[ATT_QB][ATT_CH];
  __shared__ float st_s[ATT_QB][2];
  const int c = blockIdx.x, kh = blockIdx.y, qb = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int nq = G * a.M;
  const int q0 = qb * ATT_QB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const KT* kc = reinterpret_cast<const KT*>(a.kc) + (size_t)kh * a.max_seq * HD;
  const KT* vc = reinterpret_cast<const KT*>(a.vc) + (size_t)kh * a.max_seq * HD;
  const int u0 = c * ATT_CH;

  for (int i = tid; i < ATT_CH * HD; i += ATT_THREADS) {
    const int u = i / HD, dd = i % HD;
    const int pos = u0 + u;
    kv_s[u][dd] = (pos < a.max_seq) ? ld_elem<KT>(kc, (size_t)pos * HD + dd) : 0.f;
  }
  for (int i = tid; i < ATT_QB * HD; i += ATT_THREADS) {
    const int qi = i / HD, dd = i % HD;
    const int gq = q0 + qi;
    float v = 0.f;
    if (gq < nq) {
      const int m = gq / G, h = kh * G + gq % G;
      v = a.qrot[((size_t)m * a.Hq + h) * HD + dd];
    }
    q_s[qi][dd] = v;
  }
  __syncthreads();
  // scores: lane = key, wave handles queries wave, wave+4, ...
  {
    const int u = lane;
    const int pos = u0 + u;
    for (int qi = wave; qi < ATT_QB; qi += ATT_THREADS / 64) {
      const int gq = q0 + qi;
      float s = -INFINITY;
      if (gq < nq) {
        const int m = gq / G;
        const int lim = a.lim_base + m * a.lim_step;
        const int wo = pos - a.wbase;
        const bool vis = pos < lim || (wo >= 0 && wo < 32 && ((a.wmask >> wo) & 1u));
        if (vis && pos < a.max_seq) {
          float dot = 0.f;
#pragma unroll 8
          for (int dd = 0; dd < HD; ++dd) dot = fmaf(q_s[qi][dd], kv_s[u][dd], dot);
          s = __fmul_rn(dot, a.scale);
        }
      }
      const float mx = wave_max(s);
      const float e = (s == -INFINITY) ? 0.f : expf(__fsub_rn(s, mx));
      const float l = wave_sum(e);
      p_s[qi][u] = e;
      if (lane == 0) { st_s[qi][0] = mx; st_s[qi][1] = l; }
    }
  }
  __syncthreads();
  for (int i = tid; i < ATT_CH * HD; i += ATT_THREADS) {
    const int u = i / HD, dd = i % HD;
    const int pos = u0 + u;
    kv_s[u][dd] = (pos < a.max_seq) ? ld_elem<KT>(vc, (size_t)pos * HD + dd) : 0.f;
  }
  __syncthreads();
  for (int i = tid; i < ATT_QB * HD; i += ATT_THREADS) {
    const int qi = i / HD, dd = i % HD;
    const int gq = q0 + qi;
    if (gq >= nq) continue;
    float acc = 0.f;
#pragma unroll 8
    for (int u = 0; u < ATT_CH; ++u) acc = fmaf(p_s[qi][u], kv_s[u][dd], acc);
    const int m = gq / G, h = kh * G + gq % G;
    float* out = a.part + (((size_t)m * a.Hq + h) * a.nch_max + c) * (HD + 2);
    out[dd] = acc;
    if (dd == 0) { out[HD] = st_s[qi][0]; out[HD + 1] = st_s[qi][1]; }
  }
}

// Merge the chunk partials of each (row, head) in chunk order, then (for
// layer-selection rows) the row's own key/value; o[m][h*hd + d].
template <int HD>
__global__ __launch_bounds__(HD) void k_attn_combine(const float* __restrict__ part, int nch, int nch_max,
                                                     int Hq, int Hkv, const float* __restrict__ qrot,
                                                     const float* __restrict__ selfkv, float scale,
                                                     float* __restrict__ o) {
  __shared__ float red[HD / 64 > 0 ? HD / 64 : 1];
  const int m = blockIdx.x / Hq, h = blockIdx.x % Hq;
  const int dd = threadIdx.x;
  const float* p = part + ((size_t)m * Hq + h) * nch_max * (HD + 2);
  float M = -INFINITY, L = 0.f, acc = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float* pc = p + (size_t)c * (HD + 2);
    const float lc = pc[HD + 1];
    if (lc == 0.f) continue;
    const float mc = pc[HD];
    const float Mn = fmaxf(M, mc);
    const float fa = (M == -INFINITY) ? 0.f : expf(__fsub_rn(M, Mn));
    const float fb = expf(__fsub_rn(mc, Mn));
    acc = __fadd_rn(__fmul_rn(acc, fa), __fmul_rn(pc[dd], fb));
    L = __fadd_rn(__fmul_rn(L, fa), __fmul_rn(lc, fb));
    M = Mn;
  }
  if (selfkv) {
    const int G = Hq / Hkv, kh = h / G;
    const float* k = selfkv + (((size_t)m * 2 + 0) * Hkv + kh) * HD;
    const float* v = selfkv + (((size_t)m * 2 + 1) * Hkv + kh) * HD;
    const float* q = qrot + ((size_t)m * Hq + h) * HD;
    const float s = __fmul_rn(block_sum(__fmul_rn(q[dd], k[dd]), red), scale);
    const float Mn = fmaxf(M, s);
    const float fa = (M == -INFINITY) ? 0.f : expf(__fsub_rn(M, Mn));
    const float fb = expf(__fsub_rn(s, Mn));
    acc = __fadd_rn(__fmul_rn(acc, fa), __fmul_rn(v[dd], fb));
    L = __fadd_rn(__fmul_rn(L, fa), fb);
    M = Mn;
  }
  o[((size_t)m * Hq + h) * HD + dd] = __fdiv_rn(acc, L);
}

// ---------------------------------------------------------------- LM head reduce / accept
struct HeadRes {                 // device result block, mirrored to the host
  int32_t n, bonus, argmax[64];
  float pmax[64];
};

// Per row: argmax over the tile partials (lowest index on ties) and the
// top-1 softmax probability 1 / sum_j exp(z_j - z_max).
__global__ __launch_bounds__(256) void k_head_reduce(const float* __restrict__ part, int ntile,
                                                     HeadRes* __restrict__ res, int row0) {
  __shared__ float redf[4];
  __shared__ float bm[4];
  __shared__ int bi[4];
  const int m = blockIdx.x;
  const float* p = part + (size_t)m * ntile * 3;
  float mx = -INFINITY;
  int idx = 0x7fffffff;
  for (int w = threadIdx.x; w < ntile; w += blockDim.x) {
    const float v = p[w * 3];
    const int i = __float_as_int(p[w * 3 + 1]);
    if (v > mx || (v == mx && i < idx)) { mx = v; idx = i; }
  }
  for (int o = 32; o >= 1; o >>= 1) {
    const float om = __shfl_xor(mx, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (om > mx || (om == mx && oi < idx)) { mx = om; idx = oi; }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) { bm[wv] = mx; bi[wv] = idx; }
  __syncthreads();
  mx = bm[0]; idx = bi[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i)
    if (bm[i] > mx || (bm[i] == mx && bi[i] < idx)) { mx = bm[i]; idx = bi[i]; }
  float s = 0.f;
  for (int w = threadIdx.x; w < ntile; w += blockDim.x)
    s = __fadd_rn(s, __fmul_rn(p[w * 3 + 2], expf(__fsub_rn(p[w * 3], mx))));
  s = block_sum(s, redf);
  if (threadIdx.x == 0) {
    res->argmax[row0 + m] = idx;
    res->pmax[row0 + m] = __fdiv_rn(1.0f, s);
  }
}

// Draft step bookkeeping: the drafted token becomes the next window input.
__global__ void k_draft_commit(HeadRes* res, int slot, int32_t* tok) {
  tok[slot + 1] = res->argmax[slot];
}

// Greedy acceptance: n = first i with argmax_i != draft_{i+1}; bonus =
// argmax_n; the bonus becomes the pending token tok[0].
__global__ void k_accept(HeadRes* res, int k, int32_t* tok) {
  int n = 0;
  while (n < k && res->argmax[n] == tok[n + 1]) ++n;
  res->n = n;
  res->bonus = res->argmax[n];
  tok[0] = res->argmax[n];
}

// Copy the residual states of verify row res->n (or `row` if res == nullptr)
// into the layer-selection target [L+1][d].
__global__ void k_gather_target(const float* __restrict__ hs, int rows_stride, int d, const HeadRes* res,
                                int row, float* __restrict__ target) {
  const int l = blockIdx.x;
  const int rr = res ? res->n : row;
  const float* src = hs + ((size_t)l * rows_stride + rr) * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) target[(size_t)l * d + i] = src[i];
}

// ---------------------------------------------------------------- layer-selection DP
// Stage i (layer i-1): for each j in [lo_i, hi_i] compare the executed
// candidate ex[j - ex_lo] (valid iff j in [ex_lo, ex_hi]) and the skipped
// candidate gp[j - 1 - lo_p] (valid iff j-1 in [lo_p, hi_p]) by cosine
// similarity with the target state H; keep the skip only if strictly better.
__global__ __launch_bounds__(256) void k_dp_select(const float* __restrict__ ex, int ex_lo, int ex_hi,
                                                   const float* __restrict__ gp, int lo_p, int hi_p,
                                                   const float* __restrict__ H, int d, int lo_i,
                                                   float* __restrict__ gn, float* __restrict__ dec) {
  __shared__ float red[4];
  __shared__ int take_s;
  const int j = lo_i + blockIdx.x;
  const bool eok = j >= ex_lo && j <= ex_hi;
  const bool sok = (j - 1) >= lo_p && (j - 1) <= hi_p;
  const float* e = eok ? ex + (size_t)(j - ex_lo) * d : nullptr;
  const float* s = sok ? gp + (size_t)(j - 1 - lo_p) * d : nullptr;
  float hh = 0.f, eh = 0.f, ee = 0.f, sh = 0.f, ss = 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    const float hv = H[i];
    hh = fmaf(hv, hv, hh);
    if (eok) { const float v = e[i]; eh = fmaf(v, hv, eh); ee = fmaf(v, v, ee); }
    if (sok) { const float v = s[i]; sh = fmaf(v, hv, sh); ss = fmaf(v, v, ss); }
  }
  hh = block_sum(hh, red);
  eh = block_sum(eh, red);
  ee = block_sum(ee, red);
  sh = block_sum(sh, red);
  ss = block_sum(ss, red);
  const float nh = __fsqrt_rn(hh);
  const float ce = eok ? __fdiv_rn(eh, __fmul_rn(__fsqrt_rn(ee), nh)) : NAN;
  const float cs = sok ? __fdiv_rn(sh, __fmul_rn(__fsqrt_rn(ss), nh)) : NAN;
  if (threadIdx.x == 0) {
    const int take = sok && (!eok || cs > ce);
    take_s = take;
    dec[(size_t)j * 3 + 0] = (float)take;
    dec[(size_t)j * 3 + 1] = cs;
    dec[(size_t)j * 3 + 2] = ce;
  }
  __syncthreads();
  const float* src = take_s ? s : e;
  float* dst = gn + (size_t)(j - lo_i) * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) dst[i] = src[i];
}

}  // namespace lss
