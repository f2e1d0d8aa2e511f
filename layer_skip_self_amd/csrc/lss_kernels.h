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
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

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

// Cross-lane reductions without LDS traffic.  Inside each 16-lane row four
// DPP steps pair lane i with i ^ 1, i ^ 2, the mirrored lane of its 8-lane
// half and the mirrored lane of the row; after them every lane of a row
// holds the same row result (a + b == b + a).  Wave results then combine
// the four row results (lanes 0, 16, 32, 48) as (r0 . r1) . (r2 . r3).
// Callers run them with the whole row / wave active.
template <int CTRL> __device__ __forceinline__ float dpp_t(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
#define LSS_DPP_XOR1 0xB1     // quad_perm [1, 0, 3, 2]
#define LSS_DPP_XOR2 0x4E     // quad_perm [2, 3, 0, 1]
#define LSS_DPP_HMIRROR 0x141 // row_half_mirror
#define LSS_DPP_MIRROR 0x140  // row_mirror
#define LSS_DPP_ROR8 0x128    // row_ror:8 (lane i and i ^ 8 of a row)
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// fixed-order sum over the 16 lanes of a row
__device__ __forceinline__ float sum16(float v) {
  v = __fadd_rn(v, dpp_t<LSS_DPP_XOR1>(v));
  v = __fadd_rn(v, dpp_t<LSS_DPP_XOR2>(v));
  v = __fadd_rn(v, dpp_t<LSS_DPP_HMIRROR>(v));
  v = __fadd_rn(v, dpp_t<LSS_DPP_MIRROR>(v));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  return __fadd_rn(__fadd_rn(readlane_f(v, 0), readlane_f(v, 16)), __fadd_rn(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_t<LSS_DPP_XOR1>(v));
  v = fmaxf(v, dpp_t<LSS_DPP_XOR2>(v));
  v = fmaxf(v, dpp_t<LSS_DPP_HMIRROR>(v));
  v = fmaxf(v, dpp_t<LSS_DPP_MIRROR>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
// Transposed wave sums: the totals over the 64 lanes of V values per lane
// (V a power of two, 1 <= V <= 64) with the pairing tree of wave_sum, level s
// adding lanes that differ in bit s of the lane id: quad_perm xor 1 and
// xor 2, row_half_mirror (flips bits 0-2), row_ror:8, permlane16_swap,
// permlane32_swap.  While a lane still holds more than one value, a level
// halves the list: the lane keeps one half and adds its partner's copy of
// that half (one add per kept value instead of a full tree per value).  The
// half a lane keeps at level s is k_s = bit s of its id, except
// k_0 = b0 ^ b2 and k_1 = b1 ^ b2, so that the lanes row_half_mirror pairs
// hold the same values.  Every add has the operands of the matching add in
// wave_sum, so each total is the same bit for bit.  Afterwards v[0] of
// lane l is the total of value wst_index<V>(l); lanes 0 .. V - 1 hold every
// value once.
template <int V> __device__ __forceinline__ int wst_index(int l) {
  const int b2 = (l >> 2) & 1;
  const int k[6] = {(l & 1) ^ b2, ((l >> 1) & 1) ^ b2, b2, (l >> 3) & 1, (l >> 4) & 1, (l >> 5) & 1};
  int j = 0, h = V;
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    if (h > 1) {
      h >>= 1;
      j += k[s] * h;
    }
  }
  return j;
}
template <int CTRL, int N, int V> __device__ __forceinline__ void wst_dpp(float (&v)[V], bool k) {
  if constexpr (N == 1) {
    v[0] = __fadd_rn(v[0], dpp_t<CTRL>(v[0]));
  } else {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float a = v[i], b = v[i + N / 2];
      v[i] = __fadd_rn(k ? b : a, dpp_t<CTRL>(k ? a : b));
    }
  }
}
template <bool P32> __device__ __forceinline__ float swap_add(float a, float b) {
  if constexpr (P32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __fadd_rn(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __fadd_rn(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
}
// levels 4 / 5: swap(a, b) leaves a's rows (halves) with an even bit 4 (5)
// and b's rows with an odd one; a + b is then the kept half's partial sum
template <int N, int V, bool P32> __device__ __forceinline__ void wst_swap(float (&v)[V]) {
  if constexpr (N == 1) {
    v[0] = swap_add<P32>(v[0], v[0]);
  } else {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) v[i] = swap_add<P32>(v[i], v[i + N / 2]);
  }
}
template <int V> __device__ __forceinline__ void wave_sum_t(float (&v)[V]) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "1 .. 64 values, a power of two");
  const int l = threadIdx.x & 63;
  const int b2 = (l >> 2) & 1;
  wst_dpp<LSS_DPP_XOR1, V, V>(v, ((l & 1) ^ b2) != 0);
  wst_dpp<LSS_DPP_XOR2, (V >= 2 ? V / 2 : 1), V>(v, (((l >> 1) & 1) ^ b2) != 0);
  wst_dpp<LSS_DPP_HMIRROR, (V >= 4 ? V / 4 : 1), V>(v, b2 != 0);
  wst_dpp<LSS_DPP_ROR8, (V >= 8 ? V / 8 : 1), V>(v, ((l >> 3) & 1) != 0);
  wst_swap<(V >= 16 ? V / 16 : 1), V, false>(v);
  wst_swap<(V >= 32 ? V / 32 : 1), V, true>(v);
}
// (value, index) maximum with the lowest index on ties: a total order, so the
// result does not depend on the reduction tree
__device__ __forceinline__ void argmax_merge(float& mx, int& idx, float om, int oi) {
  if (om > mx || (om == mx && oi < idx)) { mx = om; idx = oi; }
}
template <int CTRL> __device__ __forceinline__ void argmax_dpp_step(float& mx, int& idx) {
  const float om = dpp_t<CTRL>(mx);
  const int oi = dpp_i<CTRL>(idx);
  argmax_merge(mx, idx, om, oi);
}
__device__ __forceinline__ void argmax16(float& mx, int& idx) {
  argmax_dpp_step<LSS_DPP_XOR1>(mx, idx);
  argmax_dpp_step<LSS_DPP_XOR2>(mx, idx);
  argmax_dpp_step<LSS_DPP_HMIRROR>(mx, idx);
  argmax_dpp_step<LSS_DPP_MIRROR>(mx, idx);
}
__device__ __forceinline__ void argmax_wave(float& mx, int& idx) {
  argmax16(mx, idx);
  float m0 = readlane_f(mx, 0);
  int i0 = __builtin_amdgcn_readlane(idx, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) argmax_merge(m0, i0, readlane_f(mx, 16 * r), __builtin_amdgcn_readlane(idx, 16 * r));
  mx = m0;
  idx = i0;
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

// ---------------------------------------------------------------- projection input format
// The activation operand of every projection is written once, by the kernel
// that produces it, in the layout the MFMA loop reads:
//   bf16 weights: blocks of 8 elements {8 x bf16 hi, 8 x bf16 lo} with
//     hi = bf16(x), lo = bf16(x - hi) (exact: x - hi is representable), so the
//     activation keeps ~16 significant bits; a row of K elements is 4K bytes;
//   float32 weights: plain float32.
// Inputs of RMSNorm'd projections are stored already multiplied by the norm
// gain, together with per-16-column partial sums of squares of the raw row;
// the projection applies 1/sqrt(mean + eps) per row in its epilogue.
template <typename WT> struct AF;
template <> struct AF<uint16_t> {
  static __device__ __forceinline__ void store(void* xa, size_t row_off, int n, float x) {
    uint16_t* b = reinterpret_cast<uint16_t*>(xa) + 2 * row_off + (size_t)(n >> 3) * 16 + (n & 7);
    const uint16_t hb = f2bf(x);
    b[0] = hb;
    b[8] = f2bf(__fsub_rn(x, bf2f(hb)));
  }
  // element n of row row_off (for the layer-selection copies)
};
template <> struct AF<float> {
  static __device__ __forceinline__ void store(void* xa, size_t row_off, int n, float x) {
    reinterpret_cast<float*>(xa)[row_off + n] = x;
  }
};

// ---------------------------------------------------------------- small kernels
__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

// Projection input of a row held in registers by a 256-thread block
// (v[j] = element threadIdx.x + 256 j, d <= 8192): xo = h * g (g == nullptr:
// h) in the projection format, po[m][t] = sum of h^2 over columns
// 16t..16t+15 (fixed 16-lane tree).
#define PREP_THREADS 256
#define PREP_PER_THREAD 32
template <typename WT>
__device__ __forceinline__ void prep_vals(const float (&v)[PREP_PER_THREAD], int d, const float* g, void* xo,
                                          float* po, int m) {
#pragma unroll
  for (int j = 0; j < PREP_PER_THREAD; ++j) {
    const int i = threadIdx.x + j * PREP_THREADS;   // d is a multiple of 16: whole tiles per pass
    if (j * PREP_THREADS >= d) break;
    const float s = sum16(__fmul_rn(v[j], v[j]));
    if (i < d) {
      if (xo) AF<WT>::store(xo, (size_t)m * d, i, g ? __fmul_rn(v[j], g[i]) : v[j]);
      if (po && (i & 15) == 0) po[(size_t)m * (d >> 4) + (i >> 4)] = s;
    }
  }
}

// Every load is issued unconditionally (elements past d read element d - 1
// and are zeroed afterwards): a conditional load merged with a constant
// makes the compiler wait for it at the merge, one round trip per element.
template <typename T>
__device__ __forceinline__ void load_vals(float (&v)[PREP_PER_THREAD], const T* src, int d) {
#pragma unroll
  for (int j = 0; j < PREP_PER_THREAD; ++j) {
    const int i = threadIdx.x + j * PREP_THREADS;
    v[j] = ld_elem<T>(src, min(i, d - 1));
  }
#pragma unroll
  for (int j = 0; j < PREP_PER_THREAD; ++j)
    if (threadIdx.x + j * PREP_THREADS >= d) v[j] = 0.f;
}

// The same for 16 consecutive columns c0 .. c0 + 15 held by one thread
// (vector loads and stores): xo = x * g in the projection format and po =
// the 16 columns' sum of squares, added in the order of sum16's lane tree
// (pairs, then pairs of pairs, then the two quads of each half, then the
// halves), so the result is the 16-lane form's bit for bit.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}
template <typename WT>
__device__ __forceinline__ void prep16(const float (&x)[16], int c0, int d, const float* __restrict__ g, void* xo,
                                       float* __restrict__ po, int m) {
  if (xo) {
    float y[16];
    if (g) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 gg = *reinterpret_cast<const float4*>(g + c0 + 4 * q);
        y[4 * q] = __fmul_rn(x[4 * q], gg.x);
        y[4 * q + 1] = __fmul_rn(x[4 * q + 1], gg.y);
        y[4 * q + 2] = __fmul_rn(x[4 * q + 2], gg.z);
        y[4 * q + 3] = __fmul_rn(x[4 * q + 3], gg.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = x[i];
    }
    if constexpr (sizeof(WT) == 2) {
      // blocks of 8: {8 bf16 hi, 8 bf16 lo}, 32 bytes per block
      uint4* b = reinterpret_cast<uint4*>(reinterpret_cast<char*>(xo) + ((size_t)m * d + c0) * 4);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        float lo[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) lo[i] = __fsub_rn(y[8 * k + i], bf2f(f2bf(y[8 * k + i])));
        b[2 * k] = make_uint4(pack_bf2(y[8 * k], y[8 * k + 1]), pack_bf2(y[8 * k + 2], y[8 * k + 3]),
                              pack_bf2(y[8 * k + 4], y[8 * k + 5]), pack_bf2(y[8 * k + 6], y[8 * k + 7]));
        b[2 * k + 1] = make_uint4(pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(lo[4], lo[5]),
                                  pack_bf2(lo[6], lo[7]));
      }
    } else {
      float4* b = reinterpret_cast<float4*>(reinterpret_cast<float*>(xo) + (size_t)m * d + c0);
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
    }
  }
  if (po) {
    float p2[8], p4[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) p2[i] = __fadd_rn(__fmul_rn(x[2 * i], x[2 * i]), __fmul_rn(x[2 * i + 1], x[2 * i + 1]));
#pragma unroll
    for (int i = 0; i < 4; ++i) p4[i] = __fadd_rn(p2[2 * i], p2[2 * i + 1]);
    po[(size_t)m * (d >> 4) + (c0 >> 4)] = __fadd_rn(__fadd_rn(p4[0], p4[1]), __fadd_rn(p4[2], p4[3]));
  }
}
// 16 consecutive values of a row of T (16-byte aligned) as float
template <typename T> __device__ __forceinline__ void ld16(float (&x)[16], const T* src);
template <> __device__ __forceinline__ void ld16<float>(float (&x)[16], const float* src) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = reinterpret_cast<const float4*>(src)[q];
    x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
  }
}
template <> __device__ __forceinline__ void ld16<uint16_t>(float (&x)[16], const uint16_t* src) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint4 v = reinterpret_cast<const uint4*>(src)[q];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * q + 2 * i] = __uint_as_float(w[i] << 16);
      x[8 * q + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

template <typename WT>
__global__ __launch_bounds__(PREP_THREADS) void k_prep_rows(const float* __restrict__ h, int ldh, int d,
                                                            const float* __restrict__ g, void* xo,
                                                            float* __restrict__ po) {
  const int m = blockIdx.x;
  for (int c0 = threadIdx.x * 16; c0 < d; c0 += PREP_THREADS * 16) {
    float x[16];
    ld16<float>(x, h + (size_t)m * ldh + c0);
    prep16<WT>(x, c0, d, g, xo, po, m);
  }
}

// h[m][:] = E[id][:] (float32 residual stream) and its projection input.
template <typename WT>
__device__ __forceinline__ void embed_body(const WT* __restrict__ E, int id, int d, float* __restrict__ h,
                                           const float* __restrict__ g, void* xo, float* __restrict__ po, int m) {
  for (int c0 = threadIdx.x * 16; c0 < d; c0 += PREP_THREADS * 16) {
    float x[16];
    ld16<WT>(x, E + (size_t)id * d + c0);
    float4* hr = reinterpret_cast<float4*>(h + (size_t)m * d + c0);
#pragma unroll
    for (int q = 0; q < 4; ++q) hr[q] = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
    prep16<WT>(x, c0, d, g, xo, po, m);
  }
}
template <typename WT>
__global__ __launch_bounds__(PREP_THREADS) void k_embed(const WT* __restrict__ E, const int32_t* __restrict__ tok,
                                                        int ts, int d, float* __restrict__ h,
                                                        const float* __restrict__ g, void* xo,
                                                        float* __restrict__ po) {
  const int m = blockIdx.x;
  embed_body<WT>(E, tok[(size_t)m * ts], d, h, g, xo, po, m);
}
// rows of a batch: row m's token is tok[off[m]]
#define BATCH_ROWS_MAX 64
struct RowTok {
  int32_t off[BATCH_ROWS_MAX];
};
template <typename WT>
__global__ __launch_bounds__(PREP_THREADS) void k_embed_rows(const WT* __restrict__ E, const int32_t* __restrict__ tok,
                                                             RowTok rt, int d, float* __restrict__ h,
                                                             const float* __restrict__ g, void* xo,
                                                             float* __restrict__ po) {
  const int m = blockIdx.x;
  embed_body<WT>(E, tok[rt.off[m]], d, h, g, xo, po, m);
}

// Symmetric per-token int8 codes: inv = fl32(127 / amax) (correctly rounded),
// q = clamp(rint(x * inv), +-127).
__device__ __forceinline__ float quant_code(float x, float inv) {
  float q = rintf(__fmul_rn(x, inv));
  return fminf(fmaxf(q, -127.f), 127.f);
}

#define LSS_NORM_THREADS 256
#define LSS_NORM_PER_THREAD 32   // d_model <= 8192

// RMSNorm + dynamic int8 quantization of rows of h (the quantized draft):
// x = h / sqrt(mean(h^2) + eps) * g; codes of x in the projection format
// (xo), or as int8 (q8, the int8-weight draft), xs[m] = amax / 127.
template <typename WT>
__global__ __launch_bounds__(LSS_NORM_THREADS) void k_rmsnorm_quant(const float* __restrict__ h, int ldh,
                                                                    const float* __restrict__ g, int d, float eps,
                                                                    void* xo, float* __restrict__ xs,
                                                                    int8_t* __restrict__ q8) {
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
    if (i < d) v[j] = __fmul_rn(__fmul_rn(v[j], rstd), g[i]);
    amax = fmaxf(amax, fabsf(v[j]));
  }
  amax = block_max(amax, red);
  const float inv = amax > 0.f ? __fdiv_rn(127.0f, amax) : 0.f;
#pragma unroll
  for (int j = 0; j < LSS_NORM_PER_THREAD; ++j) {
    const int i = threadIdx.x + j * LSS_NORM_THREADS;
    if (i < d) {
      const float q = quant_code(v[j], inv);
      if (q8) q8[(size_t)m * d + i] = (int8_t)q;
      else AF<WT>::store(xo, (size_t)m * d, i, q);
    }
  }
  if (threadIdx.x == 0) xs[m] = __fdiv_rn(amax, 127.0f);
}

// Per-row int8 copy of a weight matrix [rows][k] for the int8-weight draft:
// each row is quantized with the activation rule (codes rint(w fl32(127 /
// amax)) clamped to +-127, scale amax / 127, amax = 0 gives codes 0).
template <typename WT>
__global__ __launch_bounds__(256) void k_quant_w8(const WT* __restrict__ w, int k, int8_t* __restrict__ q,
                                                 float* __restrict__ scale) {
  __shared__ float red[4];
  const size_t r = blockIdx.x;
  const WT* wr = w + r * k;
  float amax = 0.f;
  for (int i = threadIdx.x; i < k; i += blockDim.x) amax = fmaxf(amax, fabsf(ld_elem<WT>(wr, i)));
  amax = block_max(amax, red);
  const float inv = amax > 0.f ? __fdiv_rn(127.0f, amax) : 0.f;
  for (int i = threadIdx.x; i < k; i += blockDim.x) q[r * k + i] = (int8_t)quant_code(ld_elem<WT>(wr, i), inv);
  if (threadIdx.x == 0) scale[r] = __fdiv_rn(amax, 127.0f);
}

// Dynamic int8 quantization of float32 rows x[m][0..n): codes in the
// projection format (xo) or as int8 (q8, the stand-alone entry point),
// scale -> xs[m].  Used for the attention and SwiGLU outputs of a quantized
// draft layer.
template <typename WT>
__global__ __launch_bounds__(256) void k_quant_rows(const float* __restrict__ x, int ldx, int n, void* xo,
                                                   float* __restrict__ xs, int8_t* __restrict__ q8) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const float* xr = x + (size_t)m * ldx;
  float amax = 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) amax = fmaxf(amax, fabsf(xr[i]));
  amax = block_max(amax, red);
  const float inv = amax > 0.f ? __fdiv_rn(127.0f, amax) : 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const float q = quant_code(xr[i], inv);
    if (q8) q8[(size_t)m * n + i] = (int8_t)q;
    else AF<WT>::store(xo, (size_t)m * n, i, q);
  }
  if (threadIdx.x == 0) xs[m] = __fdiv_rn(amax, 127.0f);
}

// ---------------------------------------------------------------- sampling noise
// Counter-based random numbers of speculative sampling: Philox-4x64 with 10
// rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
// 1, 2, 3", SC 2011).  Entry v of the stream (seed, purpose, position) is
// word v % 4 of Philox(counter (v / 4, position, 0, 0), key (seed, purpose)).
// Its uniform is ((x >> 41) + 1/2) / 2^23 (exact in float32) and its Gumbel
// noise -log(-log u).  Purposes: the draft's draw at a draft row, the full
// model's draw at a row (prefill token, sampled step, bonus token), the
// acceptance uniform of the draft a verify row checks, and the replacement
// draw after a rejection.
enum { RNG_DRAFT = 1, RNG_TARGET = 2, RNG_ACCEPT = 3, RNG_RESIDUAL = 4 };

struct U64x4 { uint64_t v[4]; };

__device__ __forceinline__ U64x4 philox4x64(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                            uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += W0; k1 += W1; }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return {{c0, c1, c2, c3}};
}

__device__ __forceinline__ float rng_uniform(uint64_t x) {
  return __fmul_rn(__fadd_rn((float)(uint32_t)(x >> 41), 0.5f), 0x1p-23f);
}
__device__ __forceinline__ float rng_gumbel(uint64_t x) { return -logf(-logf(rng_uniform(x))); }
// the generator word of entry v of a stream
__device__ __forceinline__ uint64_t rng_word(uint64_t seed, int purpose, int pos, int v) {
  const U64x4 r = philox4x64((uint64_t)(v >> 2), (uint64_t)pos, 0ull, 0ull, seed, (uint64_t)purpose);
  const int w = v & 3;
  return w == 0 ? r.v[0] : w == 1 ? r.v[1] : w == 2 ? r.v[2] : r.v[3];
}

// ---------------------------------------------------------------- projections: shared definitions
// Projection arguments, the MFMA operand layout of the weights, and the
// output epilogue shared by the prefill GEMM and the decode GEMV.
//
// MFMA operand use (16x16x32 bf16 / 16x16x4 f32): lane l supplies A row
// (l & 15) = activation row, B column (l & 15) = weight row, over a k group
// chosen by (l >> 4).  A dot product does not depend on which k a lane holds
// as long as A and B agree, so the k of a step (GEMM_U vectors per lane) are
// assigned such that each load instruction reads 64 contiguous bytes of each
// of 16 weight rows, four loads covering 256 contiguous bytes per row.  With
// bf16 weights each 8-element vector meets the activation's hi and lo parts
// (two MFMAs); with float32 weights each 4-element vector feeds four MFMAs.
#define GEMM_U 4

enum { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };
enum { SCALE_NONE = 0, SCALE_NORM = 1, SCALE_XS = 2 };

struct GemmArgs {
  const void* w[3];      // weight segments stacked along N
  int nseg[3];           // rows per segment (multiples of 16)
  const void* w2;        // SWIGLU: up-projection weights [N][K]
  int N, K;
  const void* A; int lda; int M;   // activations in the projection format
  int scale;             // SCALE_*: per-row output scale
  const float* pin;      // SCALE_NORM: partial sums of squares [M][K/16]
  float eps;
  const float* xs;       // SCALE_XS: int8 scale per row
  float* Y; int ldy;     // float32 output (STORE, RESID, LOGITS; SWIGLU when xo == null)
  const float* R; int ldr;  // RESID: residual input
  void* xo; int ldo;     // projection-format output of the result (RESID: times go)
  const float* go;       // RESID: gain of the next RMSNorm (nullptr: 1)
  float* po;             // RESID: partial sums of squares of Y [M][N/16]
  float* part;           // LOGITS: per (row, tile) HEAD_PART floats (below)
  const int8_t* xq;      // int8 GEMV: activation codes of the row (scale xs[0]); nullptr: quantize A
  const float* gin;      // int8 GEMV quantizing A with SCALE_NORM: gain of that RMSNorm
  const float* wsc[3];   // int8 GEMV: per-row weight scales of each segment
  const float* wsc2;     // int8 GEMV, SWIGLU: scales of the up projection
  float inv_t;           // LOGITS: 1 / temperature; 0: greedy (no draws)
  uint64_t seed; int purpose; int pos0, pos_step;   // LOGITS draws: stream of row m is position pos0 + m pos_step
};

// LOGITS tile record: max of z / T, its lowest index, sum of exp(z / T - max),
// and (sampling) the max of z / T + Gumbel noise with its lowest index
#define HEAD_PART 5

template <typename WT> struct WTr;
template <> struct WTr<uint16_t> { static constexpr int EPL = 8, ANV = 2; };  // bf16: hi + lo vectors
template <> struct WTr<float> { static constexpr int EPL = 4, ANV = 1; };

// the GEMM_U weight vectors of one lane for the step at kb (the lane's k
// offset included), addresses clamped into the row
template <typename WT>
__device__ __forceinline__ void load_w(uint4 (&w)[GEMM_U], const WT* row, int kb, int K) {
  constexpr int EPL = WTr<WT>::EPL;
#pragma unroll
  for (int u = 0; u < GEMM_U; ++u) w[u] = *reinterpret_cast<const uint4*>(row + min(kb + u * 4 * EPL, K - EPL));
}


// One output element (row m, column n) of a projection.  y (and u, the
// up-projection of SWIGLU) carry the row scale already.  The 16 lanes of an
// aligned lane group hold columns 16 b .. 16 b + 15 of the same row (b = t16,
// one of n16 such column tiles) and call this together: RESID's partial sum
// of squares and LOGITS' tile max / argmax / sum of exponentials are fixed
// 16-lane trees.  RESID with pre = true takes the residual input and the
// next gain from rv / gv (loaded early by the caller) instead of reading them.
template <typename WT, int EPI>
__device__ __forceinline__ void proj_out(const GemmArgs& ga, int m, int M, int n, int cl, int t16, int n16, float y,
                                         float u, bool pre = false, float rv = 0.f, float gv = 1.f) {
  const bool ok = (m < M) && (n < ga.N);
  if constexpr (EPI == EPI_STORE) {
    if (ok) ga.Y[(size_t)m * ga.ldy + n] = y;
  } else if constexpr (EPI == EPI_RESID) {
    const float h = ok ? __fadd_rn(pre ? rv : ga.R[(size_t)m * ga.ldr + n], y) : 0.f;
    if (ok) ga.Y[(size_t)m * ga.ldy + n] = h;
    if (ga.xo && ok) AF<WT>::store(ga.xo, (size_t)m * ga.ldo, n, ga.go ? __fmul_rn(h, pre ? gv : ga.go[n]) : h);
    if (ga.po) {
      const float s2 = sum16(__fmul_rn(h, h));
      if (cl == 0 && m < M) ga.po[(size_t)m * n16 + t16] = s2;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const float sg = __fdiv_rn(y, __fadd_rn(1.0f, expf(-y)));
    const float o = __fmul_rn(sg, u);
    if (ok) {
      if (ga.xo) AF<WT>::store(ga.xo, (size_t)m * ga.ldo, n, o);
      else ga.Y[(size_t)m * ga.ldy + n] = o;
    }
  } else {  // EPI_LOGITS: store, then the tile record (HEAD_PART) of z / T
    if (ok) ga.Y[(size_t)m * ga.ldy + n] = y;
    const bool samp = ga.inv_t > 0.f;                  // uniform
    const float zt = samp ? __fmul_rn(y, ga.inv_t) : y;
    float mx = (n < ga.N) ? zt : -INFINITY;
    int idx = n;
    argmax16(mx, idx);
    float e = (n < ga.N) ? expf(__fsub_rn(zt, mx)) : 0.f;
    e = sum16(e);
    float gk = -INFINITY;
    int gi = n;
    if (samp) {
      if (n < ga.N) gk = __fadd_rn(zt, rng_gumbel(rng_word(ga.seed, ga.purpose, ga.pos0 + m * ga.pos_step, n)));
      argmax16(gk, gi);
    }
    if (cl == 0 && m < M) {
      float* p = ga.part + ((size_t)m * n16 + t16) * HEAD_PART;
      p[0] = mx;
      p[1] = __int_as_float(idx);
      p[2] = e;
      p[3] = gk;
      p[4] = __int_as_float(gi);
    }
  }
}


// ---------------------------------------------------------------- prefill / layer-selection GEMM (MFMA)
// P[s][q][m][n] = sum over K split s of X[m][k] W_q[n][k] for M <= 16 MT rows
// (q = 0, or 0/1 for the gate and up projections).  A workgroup is one
// 64-row weight tile (4 waves x 16 rows, each wave's rows in the MFMA B
// layout above) and one contiguous range of the K steps; the
// activation block of a step (all rows x 128 k, projection format) is
// staged once in LDS and shared by the 4 waves, so activations cost two
// bytes of L2 traffic per weight byte instead of eight.  Small N is split
// over K to fill the chip; k_pepi adds the splits in split order and runs
// the projection epilogue.  Used where rows need not match the decode GEMV
// bit for bit (prefill blocks, layer-selection rows).
#define PG_TN 64
#define PG_MAX_SPLIT 8

struct PgArgs {
  const void* w[3]; int nseg[3];   // weight segments stacked along N
  const void* w2;                  // up projection (NACC = 2)
  int N, K;
  const void* A; int lda; int M;   // activations in the projection format
  int S;                           // K splits (gridDim.y)
  float* part;                     // [S][NACC][M][N]
};

template <typename WT, int MT, int NACC>
__global__ __launch_bounds__(256) void k_pgemm(PgArgs pa) {
  constexpr int EPL = WTr<WT>::EPL;
  constexpr int KS = 4 * EPL * GEMM_U;                 // k per step
  constexpr int RB = KS * 4 / 16;                      // uint4 per staged row (4 bytes per element)
  constexpr int LDR = RB + 1;                          // padded LDS row (uint4)
  constexpr int ROWS = MT * 16;
  constexpr int SV = ROWS * RB / 256;                  // staged uint4 per thread
  static_assert(ROWS * RB % 256 == 0, "staging split");
  __shared__ uint4 a_s[2][ROWS * LDR];                 // double-buffered activation block

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int M = pa.M, K = pa.K;
  const int n0 = blockIdx.x * PG_TN + wave * 16;        // this wave's 16 weight rows
  int seg = 0, nloc = n0;
  while (seg < 2 && nloc >= pa.nseg[seg]) { nloc -= pa.nseg[seg]; ++seg; }
  const bool row_ok = n0 + r < pa.N;
  const WT* wrow = reinterpret_cast<const WT*>(pa.w[seg]) + (size_t)(row_ok ? nloc + r : 0) * K;
  const WT* wrow2 = (NACC == 2) ? reinterpret_cast<const WT*>(pa.w2) + (size_t)(row_ok ? n0 + r : 0) * K : nullptr;
  const int nsteps = (K + KS - 1) / KS;
  const int st0 = blockIdx.y * nsteps / pa.S, st1 = (blockIdx.y + 1) * nsteps / pa.S;
  const int kg = g * EPL;

  // activation block of a step: thread t moves uint4 t + 256 j of the
  // (rows x KS) block (4 elements each), k clamped into the row
  const char* abase = reinterpret_cast<const char*>(pa.A);
  const int lda4 = pa.lda * 4;
#define PG_SRC(j, st)                                                                                    \
  (reinterpret_cast<const u32x4_t*>(abase + (size_t)min((int)(threadIdx.x + (j) * 256) / RB, M - 1) * lda4 + \
                                  (size_t)min((st) * KS + ((int)(threadIdx.x + (j) * 256) % RB) * 4, K - 4) * 4))
#define PG_DST(j) (((int)(threadIdx.x + (j) * 256) / RB) * LDR + ((int)(threadIdx.x + (j) * 256) % RB))
  uint4 wb[2][NACC][GEMM_U];
  {
    u32x4_t av[SV];
#pragma unroll
    for (int j = 0; j < SV; ++j) av[j] = *PG_SRC(j, st0);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int kb = min(st0 + d, st1 - 1) * KS + kg;
      load_w<WT>(wb[d][0], wrow, kb, K);
      if constexpr (NACC == 2) load_w<WT>(wb[d][NACC - 1], wrow2, kb, K);
    }
#pragma unroll
    for (int j = 0; j < SV; ++j) reinterpret_cast<u32x4_t*>(a_s[0])[PG_DST(j)] = av[j];
  }
  __syncthreads();
  f32x4 acc[NACC][MT];
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s2 = st0; s2 < st1; s2 += 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {                      // d: compile-time buffer index
      const int st = s2 + d;
      if (st < st1) {                                  // workgroup-uniform
        const bool more = st + 1 < st1;
        u32x4_t av[SV];
        if (more) {
#pragma unroll
          for (int j = 0; j < SV; ++j) av[j] = *PG_SRC(j, st + 1);
        }
        const int kstep = st * KS;
        const uint4* blk = a_s[d];
#pragma unroll
        for (int u = 0; u < GEMM_U; ++u) {
          if (kstep + u * 4 * EPL >= K) break;         // wave-uniform: past the end of K
          const int c16 = (kg + u * 4 * EPL) * 4 / 16; // uint4 column of this lane's k in the block
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const uint4* ap = &blk[(t * 16 + r) * LDR + c16];
            if constexpr (sizeof(WT) == 2) {
              const bf16x8_t hi = __builtin_bit_cast(bf16x8_t, ap[0]), lo = __builtin_bit_cast(bf16x8_t, ap[1]);
#pragma unroll
              for (int q = 0; q < NACC; ++q) {
                const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, wb[d][q][u]);
                acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bw, acc[q][t], 0, 0, 0);
                acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bw, acc[q][t], 0, 0, 0);
              }
            } else {
              const uint4 a4 = ap[0];
              const float af[4] = {__uint_as_float(a4.x), __uint_as_float(a4.y), __uint_as_float(a4.z),
                                   __uint_as_float(a4.w)};
#pragma unroll
              for (int q = 0; q < NACC; ++q) {
                const float wf[4] = {__uint_as_float(wb[d][q][u].x), __uint_as_float(wb[d][q][u].y),
                                     __uint_as_float(wb[d][q][u].z), __uint_as_float(wb[d][q][u].w)};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[e], wf[e], acc[q][t], 0, 0, 0);
              }
            }
          }
        }
        if (st + 2 < st1) {                            // refill this weight buffer with step st + 2
          const int kb = (st + 2) * KS + kg;
          load_w<WT>(wb[d][0], wrow, kb, K);
          if constexpr (NACC == 2) load_w<WT>(wb[d][NACC - 1], wrow2, kb, K);
        }
        if (more) {
#pragma unroll
          for (int j = 0; j < SV; ++j) reinterpret_cast<u32x4_t*>(a_s[d ^ 1])[PG_DST(j)] = av[j];
        }
        __syncthreads();                               // next block staged; this one no longer read
      }
    }
  }
  // lane (r, g) holds D[row 16t + 4g + j][column n0 + r]
  const int n = n0 + r;
  if (n >= pa.N) return;
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = t * 16 + 4 * g + j;
        if (m < M) pa.part[(((size_t)blockIdx.y * NACC + q) * M + m) * pa.N + n] = acc[q][t][j];
      }
#undef PG_SRC
#undef PG_DST
}

// 1 / rms of M rows from their per-16-column partial sums of squares
// (fixed order: thread strides, wave tree, waves in order).
__global__ __launch_bounds__(256) void k_rstd(const float* __restrict__ pin, int T, int K, float eps,
                                             float* __restrict__ rstd) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  float v = 0.f;
  for (int t = threadIdx.x; t < T; t += 256) v = __fadd_rn(v, pin[(size_t)m * T + t]);
  v = block_sum(v, red);
  if (threadIdx.x == 0) rstd[m] = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(v, (float)K), eps)));
}

// Split sum + epilogue of k_pgemm: one workgroup per 16-column tile, thread
// (tid / 16, tid % 16) = (row in a 16-row pass, column in the tile).
template <typename WT, int EPI>
__global__ __launch_bounds__(256) void k_pepi(GemmArgs ga, const float* __restrict__ part, int S,
                                              const float* __restrict__ rstd) {
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  const int i = threadIdx.x & 15;
  const int n = blockIdx.x * 16 + i;
  const int M = ga.M;
  for (int m0 = 0; m0 < M; m0 += 16) {                 // uniform over the workgroup
    const int m = m0 + (threadIdx.x >> 4);
    const int mm = min(m, M - 1), nn = min(n, ga.N - 1);
    // all splits' partials loaded before the first add (one round trip), then
    // added in split order
    float pv[NACC][PG_MAX_SPLIT];
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int s = 0; s < PG_MAX_SPLIT; ++s)
        pv[q][s] = s < S ? part[(((size_t)s * NACC + q) * M + mm) * ga.N + nn] : 0.f;
    float y[NACC];
#pragma unroll
    for (int q = 0; q < NACC; ++q) {
      float v = pv[q][0];
#pragma unroll
      for (int s = 1; s < PG_MAX_SPLIT; ++s)
        if (s < S) v = __fadd_rn(v, pv[q][s]);
      y[q] = v;
    }
    if (ga.scale == SCALE_NORM) {
#pragma unroll
      for (int q = 0; q < NACC; ++q) y[q] = __fmul_rn(y[q], rstd[mm]);
    } else if (ga.scale == SCALE_XS) {
#pragma unroll
      for (int q = 0; q < NACC; ++q) y[q] = __fmul_rn(y[q], ga.xs[mm]);
    }
    proj_out<WT, EPI>(ga, m, M, n, i, blockIdx.x, gridDim.x, y[0], NACC == 2 ? y[NACC - 1] : 0.f);
  }
}

// ---------------------------------------------------------------- decode GEMV (vector ALU)
// Y[m][n] = sum_k X[m][k] * W[n][k] for the few rows of a draft, greedy or
// verify step.  Such a launch is bound by the weight stream, so the load
// pattern is chosen for HBM: each load instruction of a wave reads one 1 KB
// contiguous piece ("chunk") of one weight row (lane l: the 16 bytes at
// offset 16 l), with nontemporal hints since the weights are read once.
// The weight rows are cut into tiles of 16 rows (8 where the epilogue has
// no per-16-column partials: store, SwiGLU; more workgroups for the small
// q/k/v launch), and a workgroup walks a contiguous
// range of tiles (one tile when the grid has a workgroup per tile).  Its
// GV_WAVES waves take the chunks of K interleaved (wave w: chunks w, w + W,
// w + 2 W, ..., so the waves of a step read W neighbouring chunks of the same
// rows: 4-6 % faster than contiguous ranges per wave at K = 14336), and each
// wave walks every tile's rows in groups of RG rows, its chunks inside each
// group, RG x NACC 1 KB loads per step with ST steps in flight.  The steps run on across tile
// boundaries: the first loads of the next tile are in flight while the wave
// sums of the current tile go through LDS and its epilogue runs, so a
// workgroup keeps the weight stream going from its first load to its last.
// The activation rows are read once per workgroup.  A lane keeps the activation elements of its k in registers
// (float32, converted once from the projection format) and multiplies them
// with its 8 (bf16) / 4 (float32) weights in fused multiply-adds.
//
// Per (weight row n, activation row m) the arithmetic is fixed by K alone:
// lane l runs one FMA chain over k = c CH + l EPL + e for its wave's chunks
// c (ascending) and e ascending, the 64 lane values are
// summed by the fixed tree of wave_sum, and the GV_WAVES wave sums are
// added in wave order.  Nothing depends on M, on the tile or on the row group, so
// a verify row gets the same bits as a one-row greedy step.  The lane sums of
// a row group (RG x NACC x MB values) are formed together by the transposed
// reduction wave_sum_t, whose totals are those of wave_sum.
#define GV_WAVES 8
#ifndef GV_ST
#define GV_ST 2                  // weight steps in flight per wave
#endif
#define GV_MB_MAX 8              // activation rows per launch
#define GV_ACT_MAX 16            // MB x NCW: activation vectors (one chunk of one row) per lane

template <typename WT> struct GVt;
template <> struct GVt<uint16_t> { static constexpr int EPL = 8, AV = 2; };   // AV: uint4 per lane of split-bf16 x
template <> struct GVt<float> { static constexpr int EPL = 4, AV = 1; };
__host__ __device__ __forceinline__ int gv_chunk(int wbytes) { return wbytes == 2 ? 512 : 256; }

__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bytes of weights as floats
template <typename WT> __device__ __forceinline__ void unpack_w(const uint4& w, float (&f)[GVt<WT>::EPL]);
template <> __device__ __forceinline__ void unpack_w<uint16_t>(const uint4& w, float (&f)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void unpack_w<float>(const uint4& w, float (&f)[4]) {
  f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y); f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}
// activation elements of one lane from the projection format (hi + lo is exact)
template <typename WT>
__device__ __forceinline__ void unpack_x(const uint4 (&a)[GVt<WT>::AV], float (&x)[GVt<WT>::EPL]) {
  if constexpr (sizeof(WT) == 2) {
    const uint32_t h[4] = {a[0].x, a[0].y, a[0].z, a[0].w}, l[4] = {a[1].x, a[1].y, a[1].z, a[1].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __fadd_rn(__uint_as_float(h[i] << 16), __uint_as_float(l[i] << 16));
      x[2 * i + 1] = __fadd_rn(__uint_as_float(h[i] & 0xffff0000u), __uint_as_float(l[i] & 0xffff0000u));
    }
  } else {
    x[0] = __uint_as_float(a[0].x); x[1] = __uint_as_float(a[0].y);
    x[2] = __uint_as_float(a[0].z); x[3] = __uint_as_float(a[0].w);
  }
}

// MB: activation rows (M <= MB); NCW: chunks per wave the launch may need
// (>= ceil(nc / GV_WAVES)), MB * NCW <= GV_ACT_MAX.
template <typename WT, int MB, int NCW, int EPI, int TR = 16>
__global__ __launch_bounds__(64 * GV_WAVES) void k_gemv(GemmArgs ga) {
  constexpr int EPL = GVt<WT>::EPL, AV = GVt<WT>::AV, CH = 64 * EPL;
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int RG = 8 / NACC;                  // weight rows per step: 8 loads of 1 KB
  constexpr int NG = TR / RG;                   // row groups per tile
  // steps in flight per wave: one for the q/k/v and residual projections
  // (fewer registers, more resident workgroups), GV_ST for gate/up and the
  // LM head
  constexpr int ST = (EPI == EPI_STORE || EPI == EPI_RESID) ? 1 : GV_ST;
  static_assert(TR == 16 || (TR == 8 && (EPI == EPI_STORE || EPI == EPI_SWIGLU)),
                "8-row tiles only without per-16-column epilogue partials");
  constexpr int NU = NG * NCW;                  // steps per wave and tile (chunks past the range are skipped)
  static_assert(NU % ST == 0, "a tile's steps start at the same buffer of the load ring");
  static_assert(MB * NCW <= GV_ACT_MAX, "activation registers");
  __shared__ float part_s[2][GV_WAVES][NACC][MB][TR];   // by tile parity
  __shared__ float red_s[GV_WAVES][MB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = ga.M, K = ga.K;
  const int nc = (K + CH - 1) / CH;
  const int ncw = (nc - wave + GV_WAVES - 1) / GV_WAVES;  // chunks of this wave: wave + GV_WAVES i (<= NCW)
  const int ntile = (ga.N + TR - 1) / TR;
  const int tb = (int)((long)blockIdx.x * ntile / gridDim.x);           // this workgroup's tiles [tb, te)
  const int te = (int)((long)(blockIdx.x + 1) * ntile / gridDim.x);
  if (tb >= te) return;                                   // whole workgroup (grid <= tiles on the host)
  const int kl = lane * EPL;

  // weight rows of tile t: segment lookup (segments hold multiples of 16 rows)
  auto tile_rows = [&](int t, const WT* (&wr)[NACC], int& nrow) {
    const int tile0 = t * TR;
    int seg = 0, nloc = tile0;
    while (seg < 2 && nloc >= ga.nseg[seg]) { nloc -= ga.nseg[seg]; ++seg; }
    wr[0] = reinterpret_cast<const WT*>(ga.w[seg]) + (size_t)nloc * K;
    if constexpr (NACC == 2) wr[NACC - 1] = reinterpret_cast<const WT*>(ga.w2) + (size_t)tile0 * K;
    nrow = min(TR, ga.N - tile0);                          // rows of the tile inside N
  };
  // weight step u of a tile = (row group u / NCW, chunk wave + GV_WAVES (u % NCW))
  auto unit_load = [&](uint4 (&w)[RG][NACC], const WT* const (&wr)[NACC], int nrow, int u) {
    const int g = u / NCW, i = u % NCW;
    const int k = min((wave + GV_WAVES * i) * CH + kl, K - EPL);
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const size_t ro = (size_t)min(g * RG + r, nrow - 1) * K + k;
#pragma unroll
      for (int q = 0; q < NACC; ++q) w[r][q] = ld_nt16(wr[q] + ro);
    }
  };

  // (1) this wave's activation chunks (raw projection format)
  uint4 xr[NCW][MB][AV];
#pragma unroll
  for (int i = 0; i < NCW; ++i) {
    const int k = min((wave + GV_WAVES * min(i, max(ncw - 1, 0))) * CH + kl, K - EPL);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const uint4* pa = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(ga.A) +
                                                       ((size_t)min(m, M - 1) * ga.lda + k) * 4);
#pragma unroll
      for (int v = 0; v < AV; ++v) xr[i][m][v] = pa[v];
    }
  }
  // (2) RMSNorm partial sums of squares (one per thread and row), summed below
  const bool norm = ga.scale == SCALE_NORM;
  const int T = K >> 4;                                   // <= 64 * GV_WAVES
  const float* pp = norm ? ga.pin : reinterpret_cast<const float*>(ga.A);
  float pr[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) pr[m] = pp[norm ? (size_t)min(m, M - 1) * T + min((int)threadIdx.x, T - 1) : 0];
  // (3) the first weight steps
  const WT* cw[NACC];
  int cn;
  tile_rows(tb, cw, cn);
  uint4 wb[ST][RG][NACC];
#pragma unroll
  for (int u = 0; u < ST; ++u)
    if (u % NCW < ncw) unit_load(wb[u], cw, cn, u);
  __builtin_amdgcn_sched_barrier(0);
  // activations as float32; lanes past K hold zeros
  float x[NCW][MB][EPL];
#pragma unroll
  for (int i = 0; i < NCW; ++i) {
    const bool kv = (wave + GV_WAVES * i) * CH + kl < K;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      unpack_x<WT>(xr[i][m], x[i][m]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[i][m][e] = kv ? x[i][m][e] : 0.f;
    }
  }
  if (norm) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      float v = ((int)threadIdx.x < T) ? pr[m] : 0.f;
      v = wave_sum(v);
      if (lane == 0) red_s[wave][m] = v;
    }
  }

  // epilogue thread (m, i) = (tid / 16, tid % 16) -> row m, column tile0 + i
  const int em = threadIdx.x >> 4, ei = threadIdx.x & 15;
  const bool epi_thread = (int)threadIdx.x < 16 * MB && (TR == 16 || ei < TR);
  const int n16 = (ga.N + 15) / 16;
  const int wj = wst_index<RG * NACC * MB>(lane);          // the group value this lane's reduction ends with
  for (int t = tb; t < te; ++t) {
    const int par = (t - tb) & 1;
    const bool has_next = t + 1 < te;                      // uniform
    const WT* nw[NACC];
    int nn = cn;
#pragma unroll
    for (int q = 0; q < NACC; ++q) nw[q] = cw[q];
    if (has_next) tile_rows(t + 1, nw, nn);
    // RESID: the epilogue's residual input and next gain, loaded under the weight stream
    float rpre = 0.f, gpre = 1.f;
    if constexpr (EPI == EPI_RESID) {
      const int n = t * TR + ei;
      if (epi_thread && em < M && n < ga.N) {
        rpre = ga.R[(size_t)em * ga.ldr + n];
        if (ga.go) gpre = ga.go[n];
      }
    }
    float acc[RG][NACC][MB];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int g = u / NCW, i = u % NCW;
      if (i == 0) {
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
          for (int q = 0; q < NACC; ++q)
#pragma unroll
            for (int m = 0; m < MB; ++m) acc[r][q][m] = 0.f;
      }
      if (i < ncw) {                                       // wave-uniform
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
          for (int q = 0; q < NACC; ++q) {
            float wf[EPL];
            unpack_w<WT>(wb[u % ST][r][q], wf);
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
              for (int e = 0; e < EPL; ++e) acc[r][q][m] = fmaf(wf[e], x[i][m][e], acc[r][q][m]);
          }
      }
      // refill the ring: the step ST ahead, in this tile or the next
      const int un = u + ST;
      if (un < NU) {
        if (un % NCW < ncw) unit_load(wb[u % ST], cw, cn, un);
      } else if (has_next && (un - NU) % NCW < ncw) {
        unit_load(wb[u % ST], nw, nn, un - NU);
      }
      if (i == NCW - 1) {                                  // group g done: lane sums -> LDS
        float red[RG * NACC * MB];
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
          for (int q = 0; q < NACC; ++q)
#pragma unroll
            for (int m = 0; m < MB; ++m) red[(r * NACC + q) * MB + m] = acc[r][q][m];
        wave_sum_t<RG * NACC * MB>(red);
        if (lane < RG * NACC * MB) {
          const int m = wj % MB, q = (wj / MB) % NACC, r = wj / (MB * NACC);
          part_s[par][wave][q][m][g * RG + r] = red[0];
        }
      }
    }
    // one barrier per tile: the next writes to part_s[par] come after the
    // next tile's barrier, which every epilogue thread reaches only after
    // finishing this tile
    __syncthreads();
    if (epi_thread) {
      const int m = em, i = ei;
      float sc = 1.0f;
      bool scaled = false;
      if (m < M) {
        if (norm) {
          float v = red_s[0][m];
#pragma unroll
          for (int w = 1; w < GV_WAVES; ++w) v = __fadd_rn(v, red_s[w][m]);
          sc = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(v, (float)K), ga.eps)));
          scaled = true;
        } else if (ga.scale == SCALE_XS) {
          sc = ga.xs[m];
          scaled = true;
        }
      }
      float y[NACC];
#pragma unroll
      for (int q = 0; q < NACC; ++q) {
        float v = part_s[par][0][q][m][i];
#pragma unroll
        for (int w = 1; w < GV_WAVES; ++w) v = __fadd_rn(v, part_s[par][w][q][m][i]);
        y[q] = scaled ? __fmul_rn(v, sc) : v;
      }
      const int tile0 = t * TR;
      proj_out<WT, EPI>(ga, m, M, tile0 + i, i, tile0 / 16, n16, y[0], NACC == 2 ? y[NACC - 1] : 0.f,
                        EPI == EPI_RESID, rpre, gpre);
    }
#pragma unroll
    for (int q = 0; q < NACC; ++q) cw[q] = nw[q];
    cn = nn;
  }
}

// ---------------------------------------------------------------- decode GEMM (MFMA, up to 16 rows)
// Y[m][n] = sum_k X[m][k] W[n][k] for the 1 .. 16 rows of a greedy step, a
// verify pass or a draft step with bf16 weights, in one pass over the
// weights for any row count (a verify is one forward pass: CLaSp article,
// section 3).  The activations (projection format, bf16 hi + lo) are the
// MFMA A operand, the weight rows the B operand of v_mfma_f32_16x16x32_bf16:
// lane (r, g) supplies activation row r and weight row r at k group g, and
// receives D[4 g + j][r].  Rows past M are zeros and never stored.
//
// Weights are streamed in wide contiguous pieces: one load instruction reads
// 256 contiguous bytes of each of 4 weight rows (lane l: row l / 16, bytes
// 16 (l % 16)), which the memory system serves as fast as whole 1 KB rows,
// unlike the 16-row x 64-byte MFMA operand shape.  A wave writes the
// pieces of its unit (TN rows x 256 B per matrix) into a wave-private LDS
// buffer (row stride 272 B: the 16-row operand reads hit 16 distinct bank
// groups) and reads them back in the operand layout.  The activation
// operands of a unit come straight from L2 (rows < M only).
//
// Work split as in the vector GEMV: tiles of TN weight rows, a workgroup
// walks a contiguous range of tiles, its W MFMA waves split K into fixed
// contiguous ranges of 128-element pieces, and every wave walks the same
// number of units per tile (units past its range are empty) with ST units
// in flight across tile boundaries.  Per (n, m) the arithmetic is fixed by
// K alone: each wave runs one MFMA chain over its pieces in increasing k,
// 32 k per step, the hi then the lo part of the activation; the wave sums
// are added in wave order.  The MFMA's sum for one output does not depend
// on the row's place in the operand or on the other rows, so a verify row
// gets the bits of the greedy step at the same position.
#define VG_PB 256                      // bytes of one weight row per unit (128 bf16)
#define VG_RS (VG_PB + 16)             // LDS row stride of the transposition buffer
#define VG_MMAX 16

// one unit of a wave's ring: NI weight loads and the SUB activation
// operand pairs (hi, lo) of one 128-element piece of K
template <int NI, int SUB> struct VgUnit {
  uint4 w[NI];
  uint4 ah[SUB], al[SUB];
};

// weight rows of one tile: first row of each 16-row block, per matrix
// (segments hold multiples of 16 rows; blocks past N read the last block,
// whose outputs are never stored)
template <int NACC, int NB, int TN>
__device__ __forceinline__ void vg_tile_rows(const GemmArgs& ga, int t, const uint16_t* (&wr)[NACC][NB]) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int n0 = min(t * TN + b * 16, ga.N - 16);
    int seg = 0, nloc = n0;
    while (seg < 2 && nloc >= ga.nseg[seg]) { nloc -= ga.nseg[seg]; ++seg; }
    wr[0][b] = reinterpret_cast<const uint16_t*>(ga.w[seg]) + (size_t)nloc * ga.K;
    if constexpr (NACC == 2) wr[NACC - 1][b] = reinterpret_cast<const uint16_t*>(ga.w2) + (size_t)n0 * ga.K;
  }
}

// issue the loads of the unit for piece pc.  Every address is valid and no
// load is conditional (a conditional load merged with another value makes
// the compiler wait for it at the merge): lanes of rows >= M read row M - 1
// (the caller points arow_ptr there) and the steps of a ragged last piece
// past K read the row's last block; neither result is ever used.
template <int NACC, int NB, int TN, int NI, int SUB>
__device__ __forceinline__ void vg_load(VgUnit<NI, SUB>& U, const uint16_t* const (&wr)[NACC][NB], int pc, int K,
                                        int la, int lc, const char* arow_ptr, int g) {
  const int k0 = pc * 128;
  const int kw = min(k0 + lc * 8, K - 8);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = i / (TN / 4), row = (i % (TN / 4)) * 4 + la;
    U.w[i] = ld_nt16(wr[q][row >> 4] + (size_t)(row & 15) * K + kw);
  }
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    const int blk = min((k0 + 32 * s) / 8 + g, K / 8 - 1);
    const uint4* pa = reinterpret_cast<const uint4*>(arow_ptr + (size_t)blk * 32);
    U.ah[s] = pa[0];
    U.al[s] = pa[1];
  }
}

// W: MFMA waves per workgroup (plus one epilogue wave); it fixes how K is
// split, so one projection always launches with the same W
template <int EPI, int TN, int ST, int W>
__global__ __launch_bounds__(64 * (W + 1)) void k_vgemm(GemmArgs ga) {
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int NB = TN / 16;                      // 16-column operand blocks per tile
  constexpr int NI = NACC * TN / 4;                // load instructions per unit
  constexpr int SUB = VG_PB / 64;                  // 32-k MFMA steps per unit
  constexpr int RPP = 64 / TN;                     // epilogue rows per pass of the epilogue wave
  static_assert(TN == 16 || TN == 32, "tile of 16 or 32 weight rows");
  __shared__ __align__(16) char wl_s[W][NACC * TN * VG_RS];
  __shared__ float part_s[2][W][NACC][VG_MMAX][TN];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = ga.M, K = ga.K;
  const int ntile = (ga.N + TN - 1) / TN;
  const int tb = (int)((long)blockIdx.x * ntile / gridDim.x);
  const int te = (int)((long)(blockIdx.x + 1) * ntile / gridDim.x);
  if (tb >= te) return;                            // whole workgroup (grid <= tiles on the host)

  if (wave == W) {
    // ---- epilogue wave: the only wave that stores.  Loads and stores share
    // one counter on this chip, so a store among the MFMA waves' loads would
    // make every later wait for a load a wait for everything.
    const int n16 = (ga.N + 15) / 16;
    const int ei = lane % TN;
    const int npass = (M + RPP - 1) / RPP;
    // per-row output scale of this lane's rows (pass p: row p RPP + lane / TN)
    float sc[VG_MMAX / RPP];
#pragma unroll
    for (int p = 0; p < VG_MMAX / RPP; ++p)
      sc[p] = (ga.scale == SCALE_XS) ? ga.xs[min(p * RPP + lane / TN, M - 1)] : 1.0f;
    const bool norm = ga.scale == SCALE_NORM;
    const bool scaled = norm || ga.scale == SCALE_XS;
    if (norm) {
      // 1 / rms of each row from its per-16-column partial sums of squares
      // (K <= 8192: at most 8 per lane): lane l adds entries l + 64 j in
      // order, then the wave's fixed tree.  Four rows' loads are in flight
      // together; all of it overlaps the MFMA waves' first tile.
      const int T = K >> 4;
      for (int m0 = 0; m0 < M; m0 += 4) {
        float pv[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            pv[i][j] = ga.pin[(size_t)min(m0 + i, M - 1) * T + min(lane + 64 * j, T - 1)];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (lane + 64 * j < T) v = __fadd_rn(v, pv[i][j]);
          v = wave_sum(v);
          const float rs = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(v, (float)K), ga.eps)));
#pragma unroll
          for (int p = 0; p < VG_MMAX / RPP; ++p)
            if (m0 + i == p * RPP + lane / TN) sc[p] = rs;
        }
      }
    }
    // residual inputs and next-norm gains of a tile, loaded one tile ahead
    float rv[VG_MMAX / RPP], gv = 1.f;
    auto load_resid = [&](int t) {
      if constexpr (EPI == EPI_RESID) {
        const int n = min(t * TN + ei, ga.N - 1);
        gv = ga.go ? ga.go[n] : 1.f;
#pragma unroll
        for (int p = 0; p < VG_MMAX / RPP; ++p)
          rv[p] = ga.R[(size_t)min(p * RPP + lane / TN, M - 1) * ga.ldr + n];
      }
    };
    load_resid(tb);
    for (int t = tb; t < te; ++t) {
      const int par = (t - tb) & 1;
      __syncthreads();                             // the MFMA waves' partials of tile t are in part_s[par]
      const int tile0 = t * TN;
      float rcur[VG_MMAX / RPP], gcur = gv;
#pragma unroll
      for (int p = 0; p < VG_MMAX / RPP; ++p) rcur[p] = (EPI == EPI_RESID) ? rv[p] : 0.f;
      if (t + 1 < te) load_resid(t + 1);
#pragma unroll
      for (int p = 0; p < VG_MMAX / RPP; ++p) {
        if (p < npass) {                           // wave-uniform
          const int m = p * RPP + lane / TN;
          // whole 16-column groups inside N, rows inside M (uniform per 16 lanes)
          if (m < M && tile0 + (ei & ~15) < ga.N) {
            float y[NACC];
#pragma unroll
            for (int q = 0; q < NACC; ++q) {
              float v = part_s[par][0][q][m][ei];
#pragma unroll
              for (int w = 1; w < W; ++w) v = __fadd_rn(v, part_s[par][w][q][m][ei]);
              y[q] = scaled ? __fmul_rn(v, sc[p]) : v;
            }
            proj_out<uint16_t, EPI>(ga, m, M, tile0 + ei, ei & 15, (tile0 + (ei & ~15)) / 16, n16, y[0],
                                    NACC == 2 ? y[NACC - 1] : 0.f, EPI == EPI_RESID, rcur[p], gcur);
          }
        }
      }
    }
    return;
  }

  // ---- MFMA waves: loads, LDS transposition, MFMA; no global stores
  const int npc = (K + 127) >> 7;                  // 128-element pieces of a row
  const int p0 = wave * npc / W;
  const int np = (wave + 1) * npc / W - p0;        // pieces of this wave
  const int nmax = (npc + W - 1) / W;
  const int NUP = (nmax + ST - 1) / ST * ST;       // units per tile (every wave), a multiple of ST
  const int la = lane >> 4, lc = lane & 15;        // load role: row la of 4, 16-byte piece lc
  const int r = lane & 15, g = lane >> 4;          // operand role: row / column r, k group g
  char* wl = wl_s[wave];
  const char* arow_ptr = reinterpret_cast<const char*>(ga.A) + (size_t)min(r, M - 1) * ga.lda * 4;

  const uint16_t* cw[NACC][NB];
  vg_tile_rows<NACC, NB, TN>(ga, tb, cw);
  VgUnit<NI, SUB> ring[ST];
  // the piece a ring slot loads for unit u: units past the wave's range
  // re-read its last piece (an L2 hit, never used), so that every refill is
  // issued and the count of loads in flight is the same on every path
  const int plast = p0 + max(np, 1) - 1;
  // slot by slot, in order (the scheduler may not interleave the slots'
  // loads: the first unit's wait would then cover the whole ring)
#pragma unroll
  for (int d = 0; d < ST; ++d) {
    vg_load<NACC, NB, TN>(ring[d], cw, min(p0 + d, plast), K, la, lc, arow_ptr, g);
    __builtin_amdgcn_sched_barrier(0);
  }

  for (int t = tb; t < te; ++t) {
    const int par = (t - tb) & 1;
    const bool has_next = t + 1 < te;
    const uint16_t* nw[NACC][NB];
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int b = 0; b < NB; ++b) nw[q][b] = cw[q][b];
    if (has_next) vg_tile_rows<NACC, NB, TN>(ga, t + 1, nw);
    f32x4 acc[NACC][NB];
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[q][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int u0 = 0; u0 < NUP; u0 += ST) {
#pragma unroll
      for (int d = 0; d < ST; ++d) {
        const int u = u0 + d;
        if (u < np) {                              // wave-uniform
          // weights of the unit -> LDS (rows x 256 B), then the operand layout.
          // The buffer is private to the wave and LDS operations of a wave
          // complete in order, so no barrier is needed; the wavefront-scope
          // fences only keep the compiler from moving the previous unit's
          // reads past these writes or these writes past the reads below.
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const int q = i / (TN / 4), row = (i % (TN / 4)) * 4 + la;
            *reinterpret_cast<uint4*>(wl + (q * TN + row) * VG_RS + lc * 16) = ring[d].w[i];
          }
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          const int k0 = (p0 + u) * 128;
#pragma unroll
          for (int s = 0; s < SUB; ++s) {
            if (k0 + 32 * s < K) {                 // wave-uniform
              const bf16x8_t xh = __builtin_bit_cast(bf16x8_t, ring[d].ah[s]);
              const bf16x8_t xl = __builtin_bit_cast(bf16x8_t, ring[d].al[s]);
#pragma unroll
              for (int q = 0; q < NACC; ++q)
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                  const uint4 wf =
                      *reinterpret_cast<const uint4*>(wl + (q * TN + b * 16 + r) * VG_RS + s * 64 + g * 16);
                  const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, wf);
                  acc[q][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, bw, acc[q][b], 0, 0, 0);
                  acc[q][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, bw, acc[q][b], 0, 0, 0);
                }
            }
          }
        }
        // refill this ring slot, unconditionally: the unit ST ahead, in this
        // tile or the next.  After the last tile the refill only keeps the
        // count of loads in flight: every lane reads the same 16 bytes of
        // this tile's last piece (one line per instruction; re-reading whole
        // pieces would fetch them from memory again, as streamed lines leave
        // L2 first)
        const int un = u + ST;
        const bool nxt = un >= NUP && has_next;
        const bool dummy = un >= NUP && !has_next;
        const int uu = un >= NUP ? (has_next ? un - NUP : max(np, 1) - 1) : un;
        {
          const uint16_t* lw[NACC][NB];
#pragma unroll
          for (int q = 0; q < NACC; ++q)
#pragma unroll
            for (int b = 0; b < NB; ++b) lw[q][b] = nxt ? nw[q][b] : cw[q][b];
          vg_load<NACC, NB, TN>(ring[d], lw, min(p0 + uu, plast), K, dummy ? 0 : la, dummy ? 0 : lc, arow_ptr, g);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // wave partials -> LDS: lane (r, g) holds D[4 g + j][column r] of each block
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * g + j < M) part_s[par][wave][q][4 * g + j][b * 16 + r] = acc[q][b][j];
    // one barrier per tile: part_s[par] is rewritten two tiles later, after
    // the next tile's barrier, which the epilogue wave reaches only after
    // finishing this tile's epilogue
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int b = 0; b < NB; ++b) cw[q][b] = nw[q][b];
  }
}

// ---------------------------------------------------------------- int8 decode GEMV (W8A8 draft)
// One activation row against int8 weight rows with one float32 scale per row:
//   y[n] = fl32(fl32(acc_n) * fl32(s_n * s_x)),   acc_n = sum_k q[k] w[n][k],
// the integer sum exact (|acc| <= 127^2 K < 2^31).  The activation codes q
// (scale s_x) are given (xq, xs[0]), or formed by every workgroup from the
// float32 row A: x = A (SCALE_NONE) or x = A / sqrt(mean(A^2) + eps) * gin
// (SCALE_NORM, the mean from the per-16-column partial sums pin), then the
// per-token rule q = clamp(rint(x * fl32(127 / amax)), +-127), s_x =
// amax / 127.  Every workgroup computes the same codes (same inputs, fixed
// reduction order), so a separate quantization launch is not needed; the
// first weight loads are issued before that work.  Loads as in the bf16
// GEMV: one wave instruction reads one 1 KB chunk of one weight row (16
// codes per lane, nontemporal).  A workgroup owns G8_TR weight rows, two per
// wave; a wave walks all of K for its rows in batches of G8_U chunks and
// multiplies four code pairs per v_dot4.  Integer sums are exact, so
// neither the split nor the order of the lane and wave sums changes a bit.
#define G8_WAVES 8
#define G8_THREADS (64 * G8_WAVES)
#define G8_TR 16
#define G8_RW (G8_TR / G8_WAVES)     // weight rows per wave
#define G8_U 4
#define G8_KMAX 32768                // codes staged in LDS

__device__ __forceinline__ int dot16_i8(const uint4& a, const uint4& w, int acc) {
  acc = __builtin_amdgcn_sdot4((int)a.x, (int)w.x, acc, false);
  acc = __builtin_amdgcn_sdot4((int)a.y, (int)w.y, acc, false);
  acc = __builtin_amdgcn_sdot4((int)a.z, (int)w.z, acc, false);
  acc = __builtin_amdgcn_sdot4((int)a.w, (int)w.w, acc, false);
  return acc;
}
// integer sum over a wave (exact, any order)
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<LSS_DPP_XOR1>(v);
  v += dpp_i<LSS_DPP_XOR2>(v);
  v += dpp_i<LSS_DPP_HMIRROR>(v);
  v += dpp_i<LSS_DPP_MIRROR>(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}

// WT: the model's weight type (format of the projection input the epilogue
// writes for the next full-precision consumer).  XPT: activation elements
// per thread held in registers while the codes are formed (K <= XPT *
// G8_THREADS); K is a multiple of 16 and at most G8_KMAX.
template <typename WT, int EPI, int XPT>
__global__ __launch_bounds__(G8_THREADS) void k_gemv8(GemmArgs ga) {
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  __shared__ uint4 xq_s[G8_KMAX / 16];
  __shared__ int acc_s[NACC][G8_TR];
  __shared__ float red_s[2][G8_WAVES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = ga.K;
  const int nv = K >> 4;                                 // 16-code vectors of the row
  const int tile0 = blockIdx.x * G8_TR;
  int seg = 0, nloc = tile0;
  while (seg < 2 && nloc >= ga.nseg[seg]) { nloc -= ga.nseg[seg]; ++seg; }
  const int8_t* wb[NACC];
  wb[0] = reinterpret_cast<const int8_t*>(ga.w[seg]) + (size_t)nloc * K;
  if constexpr (NACC == 2) wb[NACC - 1] = reinterpret_cast<const int8_t*>(ga.w2) + (size_t)tile0 * K;
  const int nrow = min(G8_TR, ga.N - tile0);
  const int nch = (K + 1023) >> 10;
  const int kl = lane * 16;
  size_t ro[G8_RW];
#pragma unroll
  for (int r = 0; r < G8_RW; ++r) ro[r] = (size_t)min(wave + r * G8_WAVES, nrow - 1) * K;
  uint4 w[G8_U][G8_RW][NACC];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < G8_U; ++u) {
      const int k = (c0 + u) * 1024 + kl;
      const int kk = k < K ? k : 0;
#pragma unroll
      for (int r = 0; r < G8_RW; ++r)
#pragma unroll
        for (int q = 0; q < NACC; ++q) w[u][r][q] = ld_nt16(wb[q] + ro[r] + kk);
    }
  };
  load_batch(0);
  // activation codes into LDS (and the scale): one round of global loads
  // (row elements k = tid + G8_THREADS j, gains, partial sums), then 1/rms
  // and amax by block reductions, codes from registers
  float sx;
  if (ga.xq) {
    for (int v = threadIdx.x; v < nv; v += G8_THREADS) xq_s[v] = reinterpret_cast<const uint4*>(ga.xq)[v];
    sx = ga.xs[0];
  } else {
    const float* xf = reinterpret_cast<const float*>(ga.A);
    const bool norm = ga.scale == SCALE_NORM;
    float x[XPT], g[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int k = threadIdx.x + j * G8_THREADS;
      x[j] = k < K ? xf[k] : 0.f;
      g[j] = (norm && k < K) ? ga.gin[k] : 0.f;
    }
    float ps = (norm && (int)threadIdx.x < nv) ? ga.pin[threadIdx.x] : 0.f;
    if (norm) {                                          // 1/rms from the partial sums, in wave order
      ps = wave_sum(ps);
      if (lane == 0) red_s[0][wave] = ps;
      __syncthreads();
      float v = red_s[0][0];
#pragma unroll
      for (int i = 1; i < G8_WAVES; ++i) v = __fadd_rn(v, red_s[0][i]);
      const float rstd = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(v, (float)K), ga.eps)));
#pragma unroll
      for (int j = 0; j < XPT; ++j) x[j] = __fmul_rn(__fmul_rn(x[j], rstd), g[j]);
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < XPT; ++j) amax = fmaxf(amax, fabsf(x[j]));
    amax = wave_max(amax);
    if (lane == 0) red_s[1][wave] = amax;
    __syncthreads();
    amax = red_s[1][0];
#pragma unroll
    for (int i = 1; i < G8_WAVES; ++i) amax = fmaxf(amax, red_s[1][i]);
    const float inv = amax > 0.f ? __fdiv_rn(127.0f, amax) : 0.f;
    sx = __fdiv_rn(amax, 127.0f);
    int8_t* qs = reinterpret_cast<int8_t*>(xq_s);
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int k = threadIdx.x + j * G8_THREADS;
      if (k < K) qs[k] = (int8_t)(int)quant_code(x[j], inv);
    }
  }
  __syncthreads();
  int acc[G8_RW][NACC];
#pragma unroll
  for (int r = 0; r < G8_RW; ++r)
#pragma unroll
    for (int q = 0; q < NACC; ++q) acc[r][q] = 0;
  for (int c0 = 0; c0 < nch; c0 += G8_U) {
    if (c0 > 0) load_batch(c0);
#pragma unroll
    for (int u = 0; u < G8_U; ++u) {
      const int v = (c0 + u) * 64 + lane;
      const uint4 a = v < nv ? xq_s[v] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int r = 0; r < G8_RW; ++r)
#pragma unroll
        for (int q = 0; q < NACC; ++q) acc[r][q] = dot16_i8(a, w[u][r][q], acc[r][q]);
    }
  }
#pragma unroll
  for (int r = 0; r < G8_RW; ++r)
#pragma unroll
    for (int q = 0; q < NACC; ++q) {
      const int t = wave_sum_i(acc[r][q]);
      if (lane == 0) acc_s[q][wave + r * G8_WAVES] = t;
    }
  __syncthreads();
  // epilogue: lanes 0..15 of wave 0 -> columns tile0 .. tile0 + 15
  if (threadIdx.x >= 16) return;
  const int i = threadIdx.x;
  const int n = tile0 + i, il = min(i, nrow - 1);
  const float y = __fmul_rn((float)acc_s[0][il], __fmul_rn(ga.wsc[seg][nloc + il], sx));
  float u = 0.f;
  if constexpr (NACC == 2) u = __fmul_rn((float)acc_s[1][il], __fmul_rn(ga.wsc2[tile0 + il], sx));
  proj_out<WT, EPI>(ga, 0, 1, n, i, blockIdx.x, gridDim.x, y, u);
}

// ---------------------------------------------------------------- attention
// Two launches per layer: k_attention (rotary embedding of the queries and
// of this launch's new keys, KV-cache append, split-key partials) and
// k_attn_merge.
//
// Keys are cut into fixed 64-position chunks of absolute cache positions; a
// workgroup (chunk c, kv head, query block) computes, for each of its
// queries, the chunk's max score, sum of exponentials and weighted value sum.
// k_attn_merge then combines the chunks of each query in chunk order (and,
// for layer-selection rows, the row's own key/value).  The merge order
// depends only on positions, never on the rows in the launch or on timing,
// so a verify row equals the greedy step at the same position bit for bit.
// The launch boundary makes the partials visible to the merge; a merge
// inside the first kernel would need a device-scope fence per workgroup,
// and on this chip each such fence writes back the L2.
//
// Row m (position pos0 + m*pos_step) sees cache position u iff
//   u < lim_base + m*lim_step            (committed prefix / causal rows)
//   or u - wbase in [0, 32) with bit (u - wbase) of wmask set
//                                       (draft window slots this layer wrote).
// In causal/draft launches the rows' own keys/values are positions
// pos0 .. pos0+M-1: every workgroup rotates them from the projection output
// itself (rounded to the cache type), and query block 0 of the chunk that
// holds them writes them to the cache.  Layer-selection launches write
// nothing; each row's own key/value enters the merge directly.
//
// Tree launches (a token tree of width B and depth D; node (b, j) is the
// j-th token of branch b, at position pos0 + j): a verify row of depth j
// sees positions u <= pos0 + j; a draft row of depth j sees the committed
// prefix u < pos0 and pos0 + i (i <= j) where bit i of wmask is set (the
// pass over depth i ran this layer: the levels of a cascade may differ by
// depth).  Inside the chunks that hold positions pos0 + 1 .. pos0 + j the
// row's own branch's nodes 1..j stand in for the keys and values there
// (per-row substitutes), so its scores, chunk partials and merge are those
// of the plain step at pos0 + j after that branch's first j tokens, bit for
// bit.  Nodes that are rows of the launch are rotated from its projection
// output; a draft step's earlier nodes come from their cache slots.
#define ATT_CH 64
#define ATT_QB 32
#define ATT_THREADS 512

struct AttnArgs {
  const float* qkv; int ldqkv;     // [M][(Hq + 2 Hkv) hd] projection output
  const float2* cs;                // rotary cos/sin [max_seq][hd/2]
  void* kc; void* vc;              // layer cache [Hkv][max_seq][hd]
  int max_seq, Hq, Hkv, M;
  int pos0, pos_step;
  int lim_base, lim_step, wbase;
  uint32_t wmask;
  int self_kv;                     // 1: layer-selection rows (own key/value, no cache write)
  int tree;                        // 1: token-tree launch (rows below)
  int tree_D, tree_step;           // tree depth; 0: verify rows, j >= 1: draft rows of depth j
  int tree_b0;                     // draft rows: branch of row 0
  int nch, nz;                     // key chunks, query blocks in this launch
  float* part;                     // [Hkv][nz_max][nch_max][QB][hd + 2]
  int nz_max, nch_max;
  float* out;                      // [M][Hq * hd] float32 output (when xo == nullptr)
  void* xo;                        // [M][Hq * hd] projection-format output
  float scale;                     // 1/sqrt(hd)
  int64_t seq_stride;              // batched launches: bytes between two sequences' caches
};

// Batched launches (several independent sequences, each with its own cache
// block, rows, position and visibility): the launch's query blocks are the
// sequences' blocks one after the other; sequence i owns blocks
// [zs[i], zs[i + 1]) and rows [row0[i], row0[i] + M[i]) of the projection
// output, and its cache block is slot[i] (seq_stride bytes apart).
#define ATT_SEQ_MAX 16
struct AttnSeqs {
  int n;
  int zs[ATT_SEQ_MAX + 1];
  int row0[ATT_SEQ_MAX], M[ATT_SEQ_MAX], pos0[ATT_SEQ_MAX], lim_base[ATT_SEQ_MAX], wbase[ATT_SEQ_MAX];
  int nch[ATT_SEQ_MAX], slot[ATT_SEQ_MAX];
  uint32_t wmask[ATT_SEQ_MAX];
};

template <typename KT> __device__ __forceinline__ float kv_round(float v);
template <> __device__ __forceinline__ float kv_round<float>(float v) { return v; }
template <> __device__ __forceinline__ float kv_round<uint16_t>(float v) { return bf2f(f2bf(v)); }

// element i of the rotated (rotate-half) vector x at rotary row cs, from
// xi = x[i], its partner xp = x[i +- half] and the pair's (cos, sin)
__device__ __forceinline__ float rope_val(float xi, float xp, float2 c, bool low) {
  return low ? __fsub_rn(__fmul_rn(xi, c.x), __fmul_rn(xp, c.y)) : __fadd_rn(__fmul_rn(xi, c.x), __fmul_rn(xp, c.y));
}
__device__ __forceinline__ float rope_elem(const float* x, const float2* cs, int i, int half) {
  const bool low = i < half;
  const int j = low ? i + half : i - half;
  return rope_val(x[i], x[j], cs[low ? i : j], low);
}

// Token trees (width B, depth D; node j of branch b is the token at
// position pos0 + j): a verify launch has rows [pending token, branch 0
// nodes 1..D, branch 1 nodes, ...]; a draft launch of depth j has row b =
// node j of branch b.  Node (b, j) keeps its keys and values in cache slot
// pos0 + 1 + b D + (j - 1) (its verify row index), and a row of depth j sees
// positions [0, pos0 + j] with its own branch's nodes standing in for
// positions pos0 + 1 .. pos0 + j.
__device__ __forceinline__ int att_tree_depth(const AttnArgs& a, int m) {
  return a.tree_step > 0 ? a.tree_step : (m == 0 ? 0 : (m - 1) % a.tree_D + 1);
}
__device__ __forceinline__ int att_tree_branch(const AttnArgs& a, int m) {
  return a.tree_step > 0 ? a.tree_b0 + m : (m == 0 ? 0 : (m - 1) / a.tree_D);
}
// rotary position of launch row m
__device__ __forceinline__ int att_row_pos(const AttnArgs& a, int m) {
  return a.tree ? a.pos0 + att_tree_depth(a, m) : a.pos0 + m * a.pos_step;
}
// cache slot of launch row m: pos0 + m, or for a tree draft step of depth j
// pos0 + j + b D (increasing with the row either way)
__device__ __forceinline__ bool att_tree_draft(const AttnArgs& a) { return a.tree && a.tree_step > 0; }
__device__ __forceinline__ int att_row_slot(const AttnArgs& a, int m) {
  return att_tree_draft(a) ? a.pos0 + a.tree_step + (a.tree_b0 + m) * a.tree_D : a.pos0 + m;
}
// first launch row whose cache slot is >= s (M if none)
__device__ __forceinline__ int att_first_row(const AttnArgs& a, int s) {
  const int base = att_row_slot(a, 0), st = att_tree_draft(a) ? a.tree_D : 1;
  return s <= base ? 0 : min(a.M, (s - base + st - 1) / st);
}

// 4 consecutive cache elements as float
template <typename KT> __device__ __forceinline__ float4 ld4(const KT* p);
template <> __device__ __forceinline__ float4 ld4<float>(const float* p) { return *reinterpret_cast<const float4*>(p); }
template <> __device__ __forceinline__ float4 ld4<uint16_t>(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                     __uint_as_float(v.y & 0xffff0000u));
}

// Transposed sums over groups of 2^LB consecutive lanes (LB = 4: the 16-lane
// rows; LB = 5: the 32-lane halves): the levels of wave_sum_t below LB.
// Afterwards v[0] of lane l holds the group total of value wst_index<V>(l);
// with V < 2^LB the last levels add whole copies, so the lanes whose index
// in the group is below V hold every value once.
template <int V, int LB> __device__ __forceinline__ void grp_sum_t(float (&v)[V]) {
  static_assert(LB == 4 || LB == 5, "16- or 32-lane groups");
  static_assert(V >= 1 && V <= (1 << LB) && (V & (V - 1)) == 0, "a power of two, at most the group size");
  const int l = threadIdx.x & 63;
  const int b2 = (l >> 2) & 1;
  wst_dpp<LSS_DPP_XOR1, V, V>(v, ((l & 1) ^ b2) != 0);
  wst_dpp<LSS_DPP_XOR2, (V >= 2 ? V / 2 : 1), V>(v, (((l >> 1) & 1) ^ b2) != 0);
  wst_dpp<LSS_DPP_HMIRROR, (V >= 4 ? V / 4 : 1), V>(v, b2 != 0);
  wst_dpp<LSS_DPP_ROR8, (V >= 8 ? V / 8 : 1), V>(v, ((l >> 3) & 1) != 0);
  if constexpr (LB == 5) wst_swap<(V >= 16 ? V / 16 : 1), V, false>(v);
}

// The chunk's keys and values stay in the registers they are loaded into:
// thread t holds dims 4 (t % LPU) .. + 3 of positions t / LPU + UST j
// (LPU = hd / 4 lanes per position, UST = 512 / LPU, j < NV), one coalesced
// 16-byte load each.  Rows of this launch whose cache slot lies in the chunk
// replace their key (rotated at the row's position) and value there, rounded
// to the cache type; query block 0 writes them to the cache.
//
// Per query (row m, head h) and key position u of the chunk:
//   score: each lane's 4-dim partial q.x k.x + q.y k.y + q.z k.z + q.w k.w
//          (one FMA chain), then the fixed lane tree of grp_sum_t over the
//          LPU lanes of the position; scaled by 1/sqrt(hd) where visible;
//   chunk statistics: max and sum of exp(s - max) over the 64 positions by
//          wave_max / wave_sum (lane = position);
//   value sum, per dim: each thread's positions j = 0 .. NV - 1 in order
//          (one FMA chain), then the lanes of a wave that hold the same dims
//          (permlane swaps over lane bits 4 and 5 above LPU), then the 8
//          waves' partials in wave order.
// Queries run in groups of 4.  None of these orders depends on the rows in
// the launch, the query block or the group a query falls in.
template <typename KT, int HD>
struct AttLayout {
  static constexpr int LPU = HD / 4;                       // lanes per position
  static constexpr int LB = LPU == 32 ? 5 : 4;
  static constexpr int NV = ATT_CH * HD / 4 / ATT_THREADS;  // positions per thread
  static constexpr int UST = ATT_THREADS / LPU;            // position stride of a thread
  static constexpr int UPW = 64 / LPU;                      // positions per wave instruction
  static_assert(LPU == 16 || LPU == 32, "head dim 64 or 128");
  static_assert(NV * UST == ATT_CH, "a thread's positions cover the chunk");
};
#define ATT_QG 4

// tree nodes (B D) a launch may hold
#define ATT_TREE_NODES 16
template <typename KT, typename WT, int HD, bool TREE>
__device__ __forceinline__ void attention_body(const AttnArgs& a, int z, int zp) {
  using LY = AttLayout<KT, HD>;
  constexpr int LPU = LY::LPU, NV = LY::NV, UST = LY::UST, NW = ATT_THREADS / 64;
  __shared__ __align__(16) float q_s[ATT_QB][HD];
  __shared__ float s_s[ATT_QB][ATT_CH];                    // raw scores, then exp(s - max)
  __shared__ float st_s[ATT_QB][2];
  __shared__ __align__(16) float red_s[NW][ATT_QG][HD];    // per-wave value partials of a query group
  __shared__ __align__(16) float own_s[TREE ? ATT_TREE_NODES : 1][TREE ? HD : 4];   // tree: node b D + j - 1's key
  __shared__ __align__(16) float own_v[TREE ? ATT_TREE_NODES : 1][TREE ? HD : 4];   // and value
  // z: query block of the sequence, zp: its partials' slot in the launch
  const int c = blockIdx.x, kh = blockIdx.y;
  const int G = a.Hq / a.Hkv;
  const int nq = G * a.M;
  const int q0 = z * ATT_QB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u0 = c * ATT_CH;
  const int d4 = tid % LPU, ub = tid / LPU;              // dims 4 d4 .. 4 d4 + 3, positions ub + UST j
  KT* kc = reinterpret_cast<KT*>(a.kc) + (size_t)kh * a.max_seq * HD;
  KT* vc = reinterpret_cast<KT*>(a.vc) + (size_t)kh * a.max_seq * HD;

  // (1) keys and values of this thread's positions (clamped past the
  // capacity: the visibility rule never selects those positions)
  float4 kr[NV], vr[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const size_t o = (size_t)min(u0 + ub + UST * j, a.max_seq - 1) * HD + 4 * d4;
    kr[j] = ld4<KT>(kc + o);
    vr[j] = ld4<KT>(vc + o);
  }
  // (2) this launch's rows with a slot among them: their own key and value
  if (!a.self_kv) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int s = u0 + ub + UST * j;
      const int m = att_first_row(a, s);
      if (m < a.M && att_row_slot(a, m) == s) {
        const float* x = a.qkv + (size_t)m * a.ldqkv;
        const int d = 4 * d4;
        const bool low = d < HD / 2;
        const int pd = low ? d + HD / 2 : d - HD / 2;
        const float4 xk = *reinterpret_cast<const float4*>(x + (size_t)(a.Hq + kh) * HD + d);
        const float4 xp = *reinterpret_cast<const float4*>(x + (size_t)(a.Hq + kh) * HD + pd);
        const float4 xv = *reinterpret_cast<const float4*>(x + (size_t)(a.Hq + a.Hkv + kh) * HD + d);
        const float2* cs = a.cs + (size_t)att_row_pos(a, m) * (HD / 2) + (low ? d : pd);
        float4 k;
        k.x = kv_round<KT>(rope_val(xk.x, xp.x, cs[0], low));
        k.y = kv_round<KT>(rope_val(xk.y, xp.y, cs[1], low));
        k.z = kv_round<KT>(rope_val(xk.z, xp.z, cs[2], low));
        k.w = kv_round<KT>(rope_val(xk.w, xp.w, cs[3], low));
        const float4 v = make_float4(kv_round<KT>(xv.x), kv_round<KT>(xv.y), kv_round<KT>(xv.z), kv_round<KT>(xv.w));
        kr[j] = k;
        vr[j] = v;
        if (z == 0) {
          const size_t o = (size_t)s * HD + d;
          st_elem<KT>(kc, o, k.x); st_elem<KT>(kc, o + 1, k.y); st_elem<KT>(kc, o + 2, k.z); st_elem<KT>(kc, o + 3, k.w);
          st_elem<KT>(vc, o, v.x); st_elem<KT>(vc, o + 1, v.y); st_elem<KT>(vc, o + 2, v.z); st_elem<KT>(vc, o + 3, v.w);
        }
      }
    }
  }
  // (3) rotated queries of this block (only rows of real queries are read later)
  const int nqb = min(ATT_QB, nq - q0);
  for (int i = tid; i < nqb * HD; i += ATT_THREADS) {
    const int qi = i / HD, dd = i % HD;
    const int gq = q0 + qi;
    const int m = gq / G, h = kh * G + gq % G;
    const int pos = att_row_pos(a, m);
    q_s[qi][dd] = rope_elem(a.qkv + (size_t)m * a.ldqkv + (size_t)h * HD, a.cs + (size_t)pos * (HD / 2), dd, HD / 2);
  }
  // tree: the keys and values of the nodes whose positions lie in this
  // chunk (rotated at their positions, rounded to the cache type)
  if constexpr (TREE) {
    const int imax = a.tree_step > 0 ? a.tree_step : a.tree_D;
    const int ilo = max(1, u0 - a.pos0), ihi = min(imax, u0 + ATT_CH - 1 - a.pos0);
    if (ilo <= ihi) {
      const int bfirst = a.tree_step > 0 ? a.tree_b0 : 0;
      const int nb = a.tree_step > 0 ? a.M : (a.M - 1) / a.tree_D;
      const int ni = ihi - ilo + 1;
      for (int t = tid; t < nb * ni * HD; t += ATT_THREADS) {
        const int dd = t % HD, r = t / HD;
        const int b = bfirst + r / ni, i = ilo + r % ni;
        const int k = b * a.tree_D + i - 1;
        if (k >= ATT_TREE_NODES) continue;
        float kv, vv;
        if (a.tree_step > 0 && i < a.tree_step) {      // an earlier draft step's node: its cache slot
          const size_t slot = (size_t)(a.pos0 + 1 + k);
          kv = ld_elem<KT>(kc, slot * HD + dd);
          vv = ld_elem<KT>(vc, slot * HD + dd);
        } else {
          const int m = a.tree_step > 0 ? b - a.tree_b0 : 1 + k;
          const float* x = a.qkv + (size_t)m * a.ldqkv;
          kv = kv_round<KT>(rope_elem(x + (size_t)(a.Hq + kh) * HD, a.cs + (size_t)(a.pos0 + i) * (HD / 2), dd,
                                      HD / 2));
          vv = kv_round<KT>(x[(size_t)(a.Hq + a.Hkv + kh) * HD + dd]);
        }
        own_s[k][dd] = kv;
        own_v[k][dd] = vv;
      }
    }
  }
  __syncthreads();
  // tree rows: positions pos0 + 1 .. pos0 + depth take the row's branch's
  // nodes (node row index, or -1 for the cache tile)
  auto node_of = [&](int m, int pos) -> int {
    if constexpr (TREE) {
      const int i = pos - a.pos0;
      return (i >= 1 && i <= att_tree_depth(a, m)) ? att_tree_branch(a, m) * a.tree_D + i - 1 : -1;
    } else {
      return -1;
    }
  };
  const int ngrp = (nqb + ATT_QG - 1) / ATT_QG;
  // (4) raw scores, a group of 4 queries at a time
  for (int g = 0; g < ngrp; ++g) {
    float4 qv[ATT_QG];
    int qm[ATT_QG];
#pragma unroll
    for (int qi = 0; qi < ATT_QG; ++qi) {
      const int qq = min(g * ATT_QG + qi, nqb - 1);
      qv[qi] = *reinterpret_cast<const float4*>(&q_s[qq][4 * d4]);
      qm[qi] = (q0 + qq) / G;
    }
    float sv[ATT_QG * NV];
#pragma unroll
    for (int qi = 0; qi < ATT_QG; ++qi)
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        float4 k = kr[j];
        if constexpr (TREE) {
          const int nd = node_of(qm[qi], u0 + ub + UST * j);
          if (nd >= 0) k = *reinterpret_cast<const float4*>(&own_s[nd][4 * d4]);
        }
        float p = __fmul_rn(qv[qi].x, k.x);
        p = fmaf(qv[qi].y, k.y, p);
        p = fmaf(qv[qi].z, k.z, p);
        p = fmaf(qv[qi].w, k.w, p);
        sv[qi * NV + j] = p;
      }
    grp_sum_t<ATT_QG * NV, LY::LB>(sv);
    const int gl = lane % LPU;                             // lane in its position group
    if (gl < ATT_QG * NV) {
      const int idx = wst_index<ATT_QG * NV>(lane);
      const int qi = idx / NV, j = idx % NV;
      if (g * ATT_QG + qi < nqb) s_s[g * ATT_QG + qi][ub + UST * j] = sv[0];
    }
  }
  __syncthreads();
  // (5) chunk statistics per query (lane = position)
  for (int qb = wave; qb < nqb; qb += NW) {                // wave-uniform
    const int u = lane, pos = u0 + u;
    const int m = (q0 + qb) / G;
    const int lim = TREE ? (a.tree_step > 0 ? a.lim_base : a.lim_base + att_tree_depth(a, m))
                         : a.lim_base + m * a.lim_step;
    const int wo = pos - a.wbase;
    const bool vis = pos < lim || (wo >= 0 && wo < 32 && ((a.wmask >> wo) & 1u));
    const float s = (vis && pos < a.max_seq) ? __fmul_rn(s_s[qb][u], a.scale) : -INFINITY;
    const float mx = wave_max(s);
    const float e = (s == -INFINITY) ? 0.f : expf(__fsub_rn(s, mx));
    const float l = wave_sum(e);
    s_s[qb][u] = e;
    if (lane == 0) { st_s[qb][0] = mx; st_s[qb][1] = l; }
  }
  __syncthreads();
  // (6) value sums, a group of 4 queries at a time
  float* part = a.part + (((size_t)kh * a.nz_max + zp) * a.nch_max + c) * ATT_QB * (HD + 2);
  for (int g = 0; g < ngrp; ++g) {
    float acc[ATT_QG * 4];
#pragma unroll
    for (int qi = 0; qi < ATT_QG; ++qi) {
      const int qq = min(g * ATT_QG + qi, nqb - 1);
      const int m = (q0 + qq) / G;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int u = ub + UST * j;
        const float p = s_s[qq][u];
        float4 v = vr[j];
        if constexpr (TREE) {
          const int nd = node_of(m, u0 + u);
          if (nd >= 0) v = *reinterpret_cast<const float4*>(&own_v[nd][4 * d4]);
        }
        float* o = acc + qi * 4;
        o[0] = j == 0 ? __fmul_rn(p, v.x) : fmaf(p, v.x, o[0]);
        o[1] = j == 0 ? __fmul_rn(p, v.y) : fmaf(p, v.y, o[1]);
        o[2] = j == 0 ? __fmul_rn(p, v.z) : fmaf(p, v.z, o[2]);
        o[3] = j == 0 ? __fmul_rn(p, v.w) : fmaf(p, v.w, o[3]);
      }
    }
    // lanes of the wave that hold the same dims: bit 5 (and bit 4 for hd 64)
    int idx0;
    if constexpr (LPU == 32) {
      wst_swap<ATT_QG * 4, ATT_QG * 4, true>(acc);
      idx0 = ((lane >> 5) & 1) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) red_s[wave][(idx0 + i) / 4][4 * d4 + (idx0 + i) % 4] = acc[i];
    } else {
      wst_swap<ATT_QG * 4, ATT_QG * 4, false>(acc);
      wst_swap<ATT_QG * 2, ATT_QG * 4, true>(acc);
      idx0 = ((lane >> 4) & 1) * 8 + ((lane >> 5) & 1) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) red_s[wave][(idx0 + i) / 4][4 * d4 + (idx0 + i) % 4] = acc[i];
    }
    __syncthreads();
    for (int t = tid; t < ATT_QG * HD; t += ATT_THREADS) {
      const int qi = t / HD, dd = t % HD;
      const int qq = g * ATT_QG + qi;
      if (qq < nqb) {
        float v = red_s[0][qi][dd];
#pragma unroll
        for (int w = 1; w < NW; ++w) v = __fadd_rn(v, red_s[w][qi][dd]);
        float* o = part + (size_t)qq * (HD + 2);
        o[dd] = v;
        if (dd == 0) { o[HD] = st_s[qq][0]; o[HD + 1] = st_s[qq][1]; }
      }
    }
    if (g + 1 < ngrp) __syncthreads();                   // red_s is rewritten by the next group
  }
}

// the arguments of sequence i of a batched launch
template <int HD>
__device__ __forceinline__ AttnArgs att_for_seq(const AttnArgs& a0, const AttnSeqs& q, int i) {
  AttnArgs a = a0;
  const int r0 = q.row0[i];
  a.qkv = a0.qkv + (size_t)r0 * a0.ldqkv;
  a.M = q.M[i];
  a.pos0 = q.pos0[i];
  a.lim_base = q.lim_base[i];
  a.wbase = q.wbase[i];
  a.wmask = q.wmask[i];
  a.nch = q.nch[i];
  a.kc = reinterpret_cast<char*>(a0.kc) + (size_t)q.slot[i] * a0.seq_stride;
  a.vc = reinterpret_cast<char*>(a0.vc) + (size_t)q.slot[i] * a0.seq_stride;
  if (a0.out) a.out = a0.out + (size_t)r0 * a0.Hq * HD;
  if (a0.xo) a.xo = reinterpret_cast<char*>(a0.xo) + (size_t)r0 * a0.Hq * HD * 4;
  return a;
}
// sequence of query block z of a batched launch (wave-uniform scan)
__device__ __forceinline__ int att_seq_of(const AttnSeqs& q, int z) {
  int i = 0;
  while (i + 1 < q.n && z >= q.zs[i + 1]) ++i;
  return i;
}

template <typename KT, typename WT, int HD, bool TREE = false>
__global__ __launch_bounds__(ATT_THREADS) void k_attention(AttnArgs a) {
  attention_body<KT, WT, HD, TREE>(a, blockIdx.z, blockIdx.z);
}
template <typename KT, typename WT, int HD>
__global__ __launch_bounds__(ATT_THREADS) void k_attention_b(AttnArgs a0, AttnSeqs q) {
  const int i = att_seq_of(q, blockIdx.z);
  const AttnArgs a = att_for_seq<HD>(a0, q, i);
  if ((int)blockIdx.x >= a.nch) return;               // whole workgroup: past this sequence's chunks
  attention_body<KT, WT, HD, false>(a, blockIdx.z - q.zs[i], blockIdx.z);
}


// Merge of the chunk partials: one workgroup of HD threads per query
// (blockIdx = (query in block, kv head, query block)).  Wave 0 reduces the
// chunk statistics with lane = chunk (nch <= 64): M = max of the chunk
// maxima over chunks that saw a key (and, for layer-selection rows, the
// row's own score), weights w_c = exp(m_c - M), normalizer
// L = sum_c l_c w_c by the fixed lane tree of wave_sum (+ the own
// key's weight).  Thread dd then adds w_c * partial_c[dd] over the chunks in
// chunk order and divides by L.  Every step depends on positions only.
#define ATT_MERGE_MAXCH 64
template <typename WT, int HD>
__device__ __forceinline__ void attn_merge_body(const AttnArgs& a, int z, int zp) {
  __shared__ float wgt[ATT_MERGE_MAXCH];
  __shared__ float st_s[2];
  const int qi = blockIdx.x, kh = blockIdx.y;
  const int G = a.Hq / a.Hkv;
  const int gq = z * ATT_QB + qi;
  if (gq >= G * a.M) return;                          // whole workgroup
  const int tid = threadIdx.x, lane = tid & 63;
  const int m = gq / G, h = kh * G + gq % G;
  const float* pb = a.part + ((size_t)kh * a.nz_max + zp) * a.nch_max * ATT_QB * (HD + 2) + (size_t)qi * (HD + 2);
  const size_t cstride = (size_t)ATT_QB * (HD + 2);
  // this thread's value partials, all chunks issued at once
  float pv[ATT_MERGE_MAXCH];
#pragma unroll
  for (int c = 0; c < ATT_MERGE_MAXCH; ++c)
    if (c < a.nch) pv[c] = pb[(size_t)c * cstride + tid];
  if (tid < 64) {
    const int c = min(lane, a.nch - 1);
    const float mc = pb[(size_t)c * cstride + HD], lc = pb[(size_t)c * cstride + HD + 1];
    const bool seen = lane < a.nch && lc != 0.f;
    float self = -INFINITY;
    if (a.self_kv) {                                   // the row's own key (rotated), scaled score
      const int pos = a.pos0 + m * a.pos_step;
      const float* qx = a.qkv + (size_t)m * a.ldqkv + (size_t)h * HD;
      const float* kx = a.qkv + (size_t)m * a.ldqkv + (size_t)(a.Hq + kh) * HD;
      const float2* cs = a.cs + (size_t)pos * (HD / 2);
      float dot = 0.f;
      for (int dd = lane; dd < HD; dd += 64)
        dot = fmaf(rope_elem(qx, cs, dd, HD / 2), rope_elem(kx, cs, dd, HD / 2), dot);
      self = __fmul_rn(wave_sum(dot), a.scale);
    }
    const float M = fmaxf(wave_max(seen ? mc : -INFINITY), self);
    const float wc = seen ? expf(__fsub_rn(mc, M)) : 0.f;
    float L = wave_sum(seen ? __fmul_rn(lc, wc) : 0.f);
    float ws = 0.f;
    if (a.self_kv) {
      ws = expf(__fsub_rn(self, M));
      L = __fadd_rn(L, ws);
    }
    if (lane < ATT_MERGE_MAXCH) wgt[lane] = wc;
    if (lane == 0) { st_s[0] = L; st_s[1] = ws; }
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < ATT_MERGE_MAXCH; ++c)
    if (c < a.nch) acc = __fadd_rn(acc, __fmul_rn(pv[c], wgt[c]));
  if (a.self_kv) {
    const float v = a.qkv[(size_t)m * a.ldqkv + (size_t)(a.Hq + a.Hkv + kh) * HD + tid];
    acc = __fadd_rn(acc, __fmul_rn(v, st_s[1]));
  }
  const float o = __fdiv_rn(acc, st_s[0]);
  if (a.xo) AF<WT>::store(a.xo, (size_t)m * a.Hq * HD, h * HD + tid, o);
  else a.out[(size_t)m * a.Hq * HD + (size_t)h * HD + tid] = o;
}
template <typename WT, int HD>
__global__ __launch_bounds__(HD) void k_attn_merge(AttnArgs a) {
  attn_merge_body<WT, HD>(a, blockIdx.z, blockIdx.z);
}
template <typename WT, int HD>
__global__ __launch_bounds__(HD) void k_attn_merge_b(AttnArgs a0, AttnSeqs q) {
  const int i = att_seq_of(q, blockIdx.z);
  attn_merge_body<WT, HD>(att_for_seq<HD>(a0, q, i), blockIdx.z - q.zs[i], blockIdx.z);
}

// ---------------------------------------------------------------- LM head reduce / accept
struct HeadRes {                 // device result block, mirrored to the host
  int32_t n, bonus, argmax[64];
  float pmax[64];
  int32_t sample[64];            // sampling: draw of each row (draft slot or verify row)
  float lse[64];                 // sampling: log-sum-exp of z / T of each verify row
  float dlse[64];                // sampling: the same for each draft slot
  int32_t emit[64];              // tokens a verify round emits: accepted drafts, then the bonus
  int32_t trow;                  // verify row whose states become the layer-selection target
};

// Per row: argmax over the tile records (lowest index on ties) and the
// top-1 softmax probability 1 / sum_j exp(z_j / T - max).  With draws
// (samp): the row's Gumbel-max draw and its log-sum-exp, the latter in
// dlse (draft slots) or lse (verify rows).
#define HEAD_RED_THREADS 1024
#define HEAD_RED_REG 8
__global__ __launch_bounds__(HEAD_RED_THREADS) void k_head_reduce(const float* __restrict__ part, int ntile,
                                                                  HeadRes* __restrict__ res, int row0, int samp,
                                                                  int draft) {
  __shared__ float redf[HEAD_RED_THREADS / 64];
  __shared__ float bm[HEAD_RED_THREADS / 64], gm[HEAD_RED_THREADS / 64];
  __shared__ int bi[HEAD_RED_THREADS / 64], gx[HEAD_RED_THREADS / 64];
  const int m = blockIdx.x;
  const float* p = part + (size_t)m * ntile * HEAD_PART;
  float mx = -INFINITY, gmx = -INFINITY;
  int idx = 0x7fffffff, gidx = 0x7fffffff;
  // this thread's first HEAD_RED_REG records, all loaded before any is used
  // (tiles w = tid + j blockDim; vocabularies up to 16 x 1024 x 16 columns)
  float rm[HEAD_RED_REG], rl[HEAD_RED_REG];
  int ri[HEAD_RED_REG];
  // (unconditional loads, tiles past ntile read the last one and are
  // neutralized afterwards: see load_vals)
#pragma unroll
  for (int j = 0; j < HEAD_RED_REG; ++j) {
    const int w = min(threadIdx.x + j * HEAD_RED_THREADS, ntile - 1);
    rm[j] = p[w * HEAD_PART];
    ri[j] = __float_as_int(p[w * HEAD_PART + 1]);
    rl[j] = p[w * HEAD_PART + 2];
  }
#pragma unroll
  for (int j = 0; j < HEAD_RED_REG; ++j)
    if (threadIdx.x + j * HEAD_RED_THREADS >= ntile) {
      rm[j] = -INFINITY;
      ri[j] = 0x7fffffff;
      rl[j] = 0.f;
    }
#pragma unroll
  for (int j = 0; j < HEAD_RED_REG; ++j) argmax_merge(mx, idx, rm[j], ri[j]);
  for (int w = threadIdx.x + HEAD_RED_REG * HEAD_RED_THREADS; w < ntile; w += blockDim.x)
    argmax_merge(mx, idx, p[w * HEAD_PART], __float_as_int(p[w * HEAD_PART + 1]));
  if (samp)
    for (int w = threadIdx.x; w < ntile; w += blockDim.x)
      argmax_merge(gmx, gidx, p[w * HEAD_PART + 3], __float_as_int(p[w * HEAD_PART + 4]));
  argmax_wave(mx, idx);
  if (samp) argmax_wave(gmx, gidx);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) { bm[wv] = mx; bi[wv] = idx; gm[wv] = gmx; gx[wv] = gidx; }
  __syncthreads();
  mx = bm[0]; idx = bi[0]; gmx = gm[0]; gidx = gx[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) {
    argmax_merge(mx, idx, bm[i], bi[i]);
    argmax_merge(gmx, gidx, gm[i], gx[i]);
  }
  float s = 0.f;                                       // tiles in the same order as before
#pragma unroll
  for (int j = 0; j < HEAD_RED_REG; ++j)
    if (threadIdx.x + j * HEAD_RED_THREADS < ntile) s = __fadd_rn(s, __fmul_rn(rl[j], expf(__fsub_rn(rm[j], mx))));
  for (int w = threadIdx.x + HEAD_RED_REG * HEAD_RED_THREADS; w < ntile; w += blockDim.x)
    s = __fadd_rn(s, __fmul_rn(p[w * HEAD_PART + 2], expf(__fsub_rn(p[w * HEAD_PART], mx))));
  s = block_sum(s, redf);
  if (threadIdx.x == 0) {
    // NaN logits win no comparison: keep the indices inside the vocabulary
    const int V = ntile * 16;
    if (idx < 0 || idx >= V) idx = 0;
    if (gidx < 0 || gidx >= V) gidx = 0;
    res->argmax[row0 + m] = idx;
    res->pmax[row0 + m] = __fdiv_rn(1.0f, s);
    if (samp) {
      res->sample[row0 + m] = gidx;
      (draft ? res->dlse : res->lse)[row0 + m] = __fadd_rn(mx, logf(s));
    }
  }
}

// Draft step bookkeeping: the drafted token (argmax, or the draw) becomes
// the next window input.
__global__ void k_draft_commit(HeadRes* res, int slot, int32_t* tok, int samp) {
  tok[slot + 1] = samp ? res->sample[slot] : res->argmax[slot];
}

// Greedy acceptance: n = first i with argmax_i != draft_{i+1}; bonus =
// argmax_n (with k = 0 and draws: the draw of row 0); the bonus becomes the
// pending token tok[0].
__global__ void k_accept(HeadRes* res, int k, int32_t* tok, int samp) {
  int n = 0;
  while (n < k && res->argmax[n] == tok[n + 1]) ++n;
  const int b = samp ? res->sample[n] : res->argmax[n];
  res->n = n;
  res->bonus = b;
  res->trow = n;
  for (int i = 0; i < n; ++i) res->emit[i] = tok[i + 1];
  res->emit[n] = b;
  tok[0] = b;
}

// Top-B tokens of one logits row (B <= TOPB_MAX), largest first, equal
// logits in index order: the tree draft's candidates, written to
// tok[1..B].  Each thread keeps the best B of its entries (a sorted list,
// compile-time indices), then B rounds of a block-wide maximum pick the
// winners; the winning thread drops its head.
#define TOPB_MAX 8
#define TOPB_THREADS 1024
__device__ __forceinline__ bool topb_before(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}
__global__ __launch_bounds__(TOPB_THREADS) void k_topb(const float* __restrict__ z, int V, int B, int ts,
                                                      int32_t* __restrict__ tok) {
  __shared__ float bm[TOPB_THREADS / 64];
  __shared__ int bi[TOPB_THREADS / 64];
  float lv[TOPB_MAX];
  int li[TOPB_MAX];
#pragma unroll
  for (int j = 0; j < TOPB_MAX; ++j) { lv[j] = -INFINITY; li[j] = 0x7fffffff; }
  for (int v = threadIdx.x; v < V; v += blockDim.x) {
    float cv = z[v];
    int ci = v;
    if (cv != cv) cv = -INFINITY;                      // NaN ranks last
#pragma unroll
    for (int j = 0; j < TOPB_MAX; ++j)                 // insert: carry the smaller one down
      if (topb_before(cv, ci, lv[j], li[j])) {
        const float tv = lv[j];
        const int ti = li[j];
        lv[j] = cv; li[j] = ci;
        cv = tv; ci = ti;
      }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int r = 0; r < B; ++r) {
    float mx = lv[0];
    int idx = li[0];
    argmax_wave(mx, idx);
    if (lane == 0) { bm[wv] = mx; bi[wv] = idx; }
    __syncthreads();
    mx = bm[0]; idx = bi[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) argmax_merge(mx, idx, bm[i], bi[i]);
    __syncthreads();
    if (threadIdx.x == 0) tok[1 + r * ts] = (idx >= 0 && idx < V) ? idx : 0;
    if (li[0] == idx) {                                // the owner drops its head
#pragma unroll
      for (int j = 0; j + 1 < TOPB_MAX; ++j) { lv[j] = lv[j + 1]; li[j] = li[j + 1]; }
      lv[TOPB_MAX - 1] = -INFINITY;
      li[TOPB_MAX - 1] = 0x7fffffff;
    }
  }
}

// A tree draft step of depth j: row b's argmax is node j + 1 of branch b,
// window slot 1 + b D + j.
__global__ void k_tree_draft_commit(const HeadRes* __restrict__ res, int B, int D, int j, int32_t* tok) {
  const int b = threadIdx.x;
  if (b < B) tok[1 + b * D + j] = res->argmax[b];
}

// Greedy acceptance of a tree of width B and depth D (rows: pending token,
// then branch b's nodes 1..D in window slots 1 + b D ..): a_0 = argmax of
// row 0; the lowest branch whose first node is a_0 is followed while its
// next node equals the argmax of the row of the last accepted one.  n =
// accepted nodes, bonus = the argmax of the last accepted node's row (a_0
// when no branch starts with a_0); trow = that row.
__global__ void k_accept_tree(HeadRes* res, int B, int D, int32_t* tok) {
  const int a0 = res->argmax[0];
  int b = -1;
  for (int i = 0; i < B && b < 0; ++i)
    if (tok[1 + i * D] == a0) b = i;
  int n = 0, row = 0;
  if (b >= 0) {
    n = 1;
    row = 1 + b * D;
    while (n < D && tok[1 + b * D + n] == res->argmax[row]) { ++n; ++row; }
  }
  const int bonus = res->argmax[row];
  for (int i = 0; i < n; ++i) res->emit[i] = tok[1 + b * D + i];
  res->emit[n] = bonus;
  res->n = n;
  res->bonus = bonus;
  res->trow = row;
  tok[0] = bonus;
}

// After a tree round: the accepted nodes' keys and values (branch b's
// slots p + 1 + b D + i - 1, rotated at p + i) become positions p + i,
// i = 1..n, in every layer (blockIdx = (layer, kv head)).  Branch 0's
// nodes are in place already; a later branch's slots all lie beyond
// p + D >= p + n, so sources and destinations never overlap.
template <typename KT>
__global__ void k_tree_kv_fix(const HeadRes* __restrict__ res, int D, KT* kc, KT* vc, int Hkv, int max_seq, int hd,
                              int p) {
  const int row = res->trow;
  if (row < 1) return;
  const int b = (row - 1) / D, n = (row - 1) % D + 1;
  if (b == 0) return;
  const size_t base = (size_t)blockIdx.x * Hkv * max_seq * hd + (size_t)blockIdx.y * max_seq * hd;
  for (int t = threadIdx.x; t < n * hd; t += blockDim.x) {
    const int i = 1 + t / hd, d = t % hd;
    const size_t dst = base + (size_t)(p + i) * hd + d, src = base + (size_t)(p + b * D + i) * hd + d;
    kc[dst] = kc[src];
    vc[dst] = vc[src];
  }
}

// Speculative-sampling acceptance (the rule that keeps the full model's
// distribution): draft i (token tok[i+1], drawn from draft logits row i at
// position pos0 + i) is accepted iff r_i q_i(d) < p_i(d), with p_i the
// softmax of verify row i at temperature T, q_i that of the draft row and
// r_i the acceptance uniform of position pos0 + i.  Lane i of every wave
// takes test i; the first rejection is the lowest rejecting lane (k if none).
__device__ __forceinline__ int spec_first_reject(const float* __restrict__ zp, const float* __restrict__ zq, int V,
                                                 const HeadRes* res, const int32_t* tok, int k, float inv_t,
                                                 uint64_t seed, int pos0) {
  const int i = threadIdx.x & 63;
  bool rej = false;
  if (i < k) {
    const int d = min(max(tok[i + 1], 0), V - 1);
    const float p = expf(__fsub_rn(__fmul_rn(zp[(size_t)i * V + d], inv_t), res->lse[i]));
    const float q = expf(__fsub_rn(__fmul_rn(zq[(size_t)i * V + d], inv_t), res->dlse[i]));
    const float r = rng_uniform(rng_word(seed, RNG_ACCEPT, pos0 + i, 0));
    rej = !(__fmul_rn(r, q) < p);
  }
  const unsigned long long mask = __ballot(rej);
  return mask ? __ffsll((long long)mask) - 1 : k;
}

// Replacement draw after the first rejection i: Gumbel-max over
// log max(0, p_i - q_i) with the replacement stream of position pos0 + i,
// and the same noise on z_i / T (used only if rounding leaves no positive
// entry).  Workgroup b covers entries [b SPEC_RES_PER_WG, ...), four
// consecutive entries (one generator block) per thread, and writes
// {max, index, fallback max, fallback index}.  Nothing runs when every
// draft is accepted.
#define SPEC_RES_THREADS 256
#define SPEC_RES_PER_WG (4 * SPEC_RES_THREADS)
__global__ __launch_bounds__(SPEC_RES_THREADS) void k_spec_residual(const float* __restrict__ zp,
                                                                    const float* __restrict__ zq, int V,
                                                                    const HeadRes* __restrict__ res,
                                                                    const int32_t* __restrict__ tok, int k,
                                                                    float inv_t, uint64_t seed, int pos0,
                                                                    float* __restrict__ out) {
  __shared__ float sm[SPEC_RES_THREADS / 64][2];
  __shared__ int si[SPEC_RES_THREADS / 64][2];
  const int i = spec_first_reject(zp, zq, V, res, tok, k, inv_t, seed, pos0);
  if (i >= k) return;                                  // uniform over the workgroup
  const float* rp = zp + (size_t)i * V;
  const float* rq = zq + (size_t)i * V;
  const float lsp = res->lse[i], lsq = res->dlse[i];
  float km = -INFINITY, fm = -INFINITY;
  int ki = 0x7fffffff, fi = 0x7fffffff;
  const int v0 = blockIdx.x * SPEC_RES_PER_WG + threadIdx.x * 4;
  if (v0 < V) {
    const U64x4 r = philox4x64((uint64_t)(v0 >> 2), (uint64_t)(pos0 + i), 0ull, 0ull, seed, RNG_RESIDUAL);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int v = v0 + w;
      if (v < V) {
        const float zpt = __fmul_rn(rp[v], inv_t);
        const float g = rng_gumbel(r.v[w]);
        const float pw = expf(__fsub_rn(zpt, lsp));
        const float qw = expf(__fsub_rn(__fmul_rn(rq[v], inv_t), lsq));
        const float wv = __fsub_rn(pw, qw);
        argmax_merge(km, ki, wv > 0.f ? __fadd_rn(logf(wv), g) : -INFINITY, v);
        argmax_merge(fm, fi, __fadd_rn(zpt, g), v);
      }
    }
  }
  argmax_wave(km, ki);
  argmax_wave(fm, fi);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) { sm[wv][0] = km; si[wv][0] = ki; sm[wv][1] = fm; si[wv][1] = fi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < SPEC_RES_THREADS / 64; ++w) {
      argmax_merge(km, ki, sm[w][0], si[w][0]);
      argmax_merge(fm, fi, sm[w][1], si[w][1]);
    }
    float* o = out + (size_t)blockIdx.x * 4;
    o[0] = km; o[1] = __int_as_float(ki); o[2] = fm; o[3] = __int_as_float(fi);
  }
}

// Round result of speculative sampling: n = first rejection; the bonus is
// the replacement draw (merged over the workgroup records in workgroup
// order) or, with every draft accepted, the draw of verify row k.
#define SPEC_FIN_THREADS 256
__global__ __launch_bounds__(SPEC_FIN_THREADS) void k_spec_final(const float* __restrict__ zp,
                                                                 const float* __restrict__ zq, int V,
                                                                 HeadRes* __restrict__ res, int32_t* tok, int k,
                                                                 float inv_t, uint64_t seed, int pos0,
                                                                 const float* __restrict__ rec, int nrec) {
  __shared__ float sm[SPEC_FIN_THREADS / 64][2];
  __shared__ int si[SPEC_FIN_THREADS / 64][2];
  const int i = spec_first_reject(zp, zq, V, res, tok, k, inv_t, seed, pos0);
  int b;
  if (i >= k) {
    b = res->sample[k];
  } else {
    float km = -INFINITY, fm = -INFINITY;
    int ki = 0x7fffffff, fi = 0x7fffffff;
    for (int w = threadIdx.x; w < nrec; w += blockDim.x) {
      argmax_merge(km, ki, rec[w * 4], __float_as_int(rec[w * 4 + 1]));
      argmax_merge(fm, fi, rec[w * 4 + 2], __float_as_int(rec[w * 4 + 3]));
    }
    argmax_wave(km, ki);
    argmax_wave(fm, fi);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (lane == 0) { sm[wv][0] = km; si[wv][0] = ki; sm[wv][1] = fm; si[wv][1] = fi; }
    __syncthreads();
    km = sm[0][0]; ki = si[0][0]; fm = sm[0][1]; fi = si[0][1];
    for (int w = 1; w < SPEC_FIN_THREADS / 64; ++w) {
      argmax_merge(km, ki, sm[w][0], si[w][0]);
      argmax_merge(fm, fi, sm[w][1], si[w][1]);
    }
    b = km > -INFINITY ? ki : fi;
    if (b < 0 || b >= V) b = 0;                        // NaN logits win no comparison
  }
  if (threadIdx.x == 0) {
    res->n = i;
    res->bonus = b;
    res->trow = i;
    for (int j = 0; j < i; ++j) res->emit[j] = tok[j + 1];
    res->emit[i] = b;
    tok[0] = b;
  }
}

// ---------------------------------------------------------------- stand-alone greedy acceptance
// The fused argmax-compare acceptance on logits the caller already holds:
// rows [k+1][V] of a verify pass and the k drafts.  k_argmax_chunks writes
// one {max, lowest index} record per (row, chunk of ACC_CH columns);
// k_accept_records reduces each row's records (the same total order, so the
// split changes nothing), then takes the greedy rule: n = length of the
// longest prefix of the drafts equal to the rows' argmaxes, bonus = argmax
// of row n.  NaN never wins a comparison; a row of NaNs yields index 0.
#define ACC_CH 4096
#define ACC_THREADS 256
struct AccRec { float mx; int idx; };

__global__ __launch_bounds__(ACC_THREADS) void k_argmax_chunks(const float* __restrict__ z, int V,
                                                              AccRec* __restrict__ rec, int nchunk) {
  __shared__ float bm[ACC_THREADS / 64];
  __shared__ int bi[ACC_THREADS / 64];
  const int c = blockIdx.x, row = blockIdx.y;
  const float* zr = z + (size_t)row * V;
  float mx = -INFINITY;
  int idx = 0x7fffffff;
  const int v0 = c * ACC_CH;
  const int v1 = min(v0 + ACC_CH, V);
  float vals[ACC_CH / ACC_THREADS];                  // all loads in flight before the compares
#pragma unroll
  for (int j = 0; j < ACC_CH / ACC_THREADS; ++j) {
    const int v = v0 + (int)threadIdx.x + j * ACC_THREADS;
    vals[j] = v < v1 ? zr[v] : -INFINITY;
  }
#pragma unroll
  for (int j = 0; j < ACC_CH / ACC_THREADS; ++j) {
    const int v = v0 + (int)threadIdx.x + j * ACC_THREADS;
    if (v < v1) argmax_merge(mx, idx, vals[j], v);
  }
  argmax_wave(mx, idx);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { bm[w] = mx; bi[w] = idx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < ACC_THREADS / 64; ++i) argmax_merge(mx, idx, bm[i], bi[i]);
    rec[(size_t)row * nchunk + c] = AccRec{mx, idx};
  }
}

// result[0] = n, result[1] = bonus, result[2 + r] = argmax of row r
__global__ __launch_bounds__(ACC_THREADS) void k_accept_records(const AccRec* __restrict__ rec, int nchunk, int rows,
                                                               int V, const int32_t* __restrict__ drafts,
                                                               int32_t* __restrict__ result) {
  __shared__ int am_s[64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int r = w; r < rows; r += ACC_THREADS / 64) {   // one wave per row, lane = chunk
    float mx = -INFINITY;
    int idx = 0x7fffffff;
    for (int c = lane; c < nchunk; c += 64) argmax_merge(mx, idx, rec[(size_t)r * nchunk + c].mx,
                                                         rec[(size_t)r * nchunk + c].idx);
    argmax_wave(mx, idx);
    if (lane == 0) am_s[r] = (idx >= 0 && idx < V) ? idx : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < rows - 1 && am_s[n] == drafts[n]) ++n;
    result[0] = n;
    result[1] = am_s[n];
  }
  for (int r = threadIdx.x; r < rows; r += ACC_THREADS) result[2 + r] = am_s[r];
}

// Copy the residual states of verify row res->trow (or `row` if res ==
// nullptr) into the layer-selection target [L+1][d].
__global__ void k_gather_target(const float* __restrict__ hs, int rows_stride, int d, const HeadRes* res,
                                int row, float* __restrict__ target) {
  const int l = blockIdx.x;
  const int rr = res ? res->trow : row;
  const float4* src = reinterpret_cast<const float4*>(hs + ((size_t)l * rows_stride + rr) * d);
  float4* dst = reinterpret_cast<float4*>(target + (size_t)l * d);
#pragma unroll 4
  for (int i = threadIdx.x; i < d / 4; i += blockDim.x) dst[i] = src[i];   // d is a multiple of 16
}

// ---------------------------------------------------------------- batches of independent sequences
// Several sequences share one pass over the weights: each keeps its own
// cache block, window, token slots (tok + seq * ts) and result block, and a
// batched head writes the rows' results into one scratch block (bres) in
// the pass's row order.  Every per-row step is the single-sequence one.

// A batched draft step: row m (sequence seq[m], window slot slot[m]) gets
// its argmax as the slot's drafted token and its top-1 probability in the
// sequence's result block.
struct BatchRows {
  int n;
  int seq[BATCH_ROWS_MAX], slot[BATCH_ROWS_MAX];
};
__global__ void k_draft_commit_b(const HeadRes* __restrict__ bres, BatchRows r, HeadRes* res, int32_t* tok, int ts) {
  const int m = threadIdx.x;
  if (m >= r.n) return;
  const int s = r.seq[m], w = r.slot[m];
  const int a = bres->argmax[m];
  tok[(size_t)s * ts + w + 1] = a;
  res[s].argmax[w] = a;
  res[s].pmax[w] = bres->pmax[m];
}

// A batched verify pass: sequence seq[i] owns rows row0[i] .. row0[i] + k[i]
// (pending token, then its k[i] drafts).  Greedy acceptance per sequence as
// k_accept; trow is the pass row of the last accepted token.
struct BatchSeqs {
  int n;
  int seq[ATT_SEQ_MAX], row0[ATT_SEQ_MAX], k[ATT_SEQ_MAX];
};
__global__ void k_accept_b(const HeadRes* __restrict__ bres, BatchSeqs b, HeadRes* res, int32_t* tok, int ts) {
  const int i = threadIdx.x;
  if (i >= b.n) return;
  HeadRes* r = res + b.seq[i];
  int32_t* t = tok + (size_t)b.seq[i] * ts;
  const int32_t* am = bres->argmax + b.row0[i];
  int n = 0;
  while (n < b.k[i] && am[n] == t[n + 1]) ++n;
  const int bonus = am[n];
  r->n = n;
  r->bonus = bonus;
  r->trow = b.row0[i] + n;
  for (int j = 0; j < n; ++j) r->emit[j] = t[j + 1];
  r->emit[n] = bonus;
  t[0] = bonus;
}

// the residual states of each sequence's trow into its layer-selection
// target (blockIdx = (layer, sequence of the pass))
__global__ void k_gather_target_b(const float* __restrict__ hs, int rows_stride, int d, const HeadRes* res,
                                  BatchSeqs b, float* __restrict__ target, size_t tstride) {
  const int l = blockIdx.x, i = blockIdx.y;
  const int rr = res[b.seq[i]].trow;
  const float4* src = reinterpret_cast<const float4*>(hs + ((size_t)l * rows_stride + rr) * d);
  float4* dst = reinterpret_cast<float4*>(target + (size_t)b.seq[i] * tstride + (size_t)l * d);
#pragma unroll 4
  for (int j = threadIdx.x; j < d / 4; j += blockDim.x) dst[j] = src[j];
}

// ---------------------------------------------------------------- layer-selection DP
// Stage i (layer i-1): for each j in [lo_i, hi_i] compare the executed
// candidate ex[j - ex_lo] (valid iff j in [ex_lo, ex_hi]) and the skipped
// candidate gp[j - 1 - lo_p] (valid iff j-1 in [lo_p, hi_p]) by cosine
// similarity with the target state H; keep the skip only if strictly better.
// The chosen state goes to gn[j - lo_i] with its projection input for the
// next layer (gain g) when xo != nullptr.
template <typename WT>
__global__ __launch_bounds__(PREP_THREADS) void k_dp_select(const float* __restrict__ ex, int ex_lo, int ex_hi,
                                                   const float* __restrict__ gp, int lo_p, int hi_p,
                                                   const float* __restrict__ H, int d, int lo_i,
                                                   float* __restrict__ gn, float* __restrict__ dec,
                                                   const float* __restrict__ g, void* xo, float* __restrict__ po) {
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
  const int row = j - lo_i;
  float* dst = gn + (size_t)row * d;
  float v[PREP_PER_THREAD];
  load_vals<float>(v, src, d);
#pragma unroll
  for (int jj = 0; jj < PREP_PER_THREAD; ++jj) {
    const int i = threadIdx.x + jj * PREP_THREADS;
    if (i < d) dst[i] = v[jj];
  }
  if (xo) prep_vals<WT>(v, d, g, xo, po, row);
}

}  // namespace lss
