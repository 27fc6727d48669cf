// Row softmax for gfx950 (MI355X): y_ij = exp(x_ij - max_j x_ij) / sum_j
// exp(x_ij - max_j x_ij) over every row of an M x N matrix -- the fused
// softmax of "4.4 Writing GPU Kernels with Triton", section "Kernel 2: Fused
// Softmax": each row is read from HBM once and written once, with the
// maximum, the exponentials and the sum formed on chip.
//
// The kernel is bound by HBM. A short row belongs to one wave (four rows per
// workgroup) and lives in its registers, so the reductions are wave-wide (no
// LDS): up to 2048 columns of 16-bit input, 1024 of fp32. Longer rows belong
// to a workgroup of 4 waves (up to 8192 16-bit or 4096 fp32 columns) or 16
// (up to 65536) and the reductions add one LDS exchange; longer rows still
// take two passes (an online maximum and sum, then the normalised write: two
// reads and one write). Loads are 16-byte
// vectors when the row pointers, the strides and N allow it, and coalesced
// element loads otherwise. Arithmetic is fp32; the exponential is
// v_exp_f32 on x * log2(e) - max * log2(e).

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"

namespace attn_internal {
void set_last_hip_error(int e);
}

namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct SmParams {
  const void *x;
  void *y;
  int64_t xs, ys;  // row strides (elements)
  int M, N;
};

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<__bf16>(__bf16 v) { return (float)v; }
template <>
__device__ __forceinline__ float to_f32<_Float16>(_Float16 v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v) { return (T)v; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Reduction over the WPR waves that share a row (WPR = 1: the wave alone;
// otherwise the workgroup is that one row).
template <int WPR, bool IS_MAX>
__device__ __forceinline__ float row_reduce(float v, float *red, int wave) {
  v = IS_MAX ? wave_max(v) : wave_sum(v);
  if constexpr (WPR > 1) {
    __syncthreads();  // the previous use of `red` is over
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < WPR; ++w) r = IS_MAX ? fmaxf(r, red[w]) : r + red[w];
    v = r;
  }
  return v;
}

// Threads per workgroup of the register-resident kernel: four one-wave rows,
// or one row of 4 or 16 waves.
template <int WPR>
constexpr int rows_threads() { return WPR == 1 ? 256 : 64 * WPR; }

// Each row of x is read once and each row of y written once by the one-pass
// kernel: with the non-temporal hint (1) on those 16-byte loads and stores,
// or plain (0).
#ifndef ATTN_CFG_SM_NONTEMPORAL
#define ATTN_CFG_SM_NONTEMPORAL 1
#endif
// Values per lane that a one- or four-wave row holds in registers, for
// fp32 and for 16-bit inputs (at most 64). Fewer values per lane send rows
// to more waves sooner, which keeps more waves per CU loading: with 16,
// fp32 rows of 1025 to 4096 columns take four waves; with 32, 16-bit rows
// of 2049 to 4096 columns do. Measured against 64 (interleaved, M x N of
// 2^27 elements): fp32 +7.0% to +7.6% at 2048 and 4096 columns, +2.2% to
// +5.2% at 8192 and 16384; bf16 +4.7% at 4096, +1.5% at 16384, equal at 512
// and 2048. 16 for 16-bit rows lost 10-18% at 2048 and 8192 columns.
#ifndef ATTN_CFG_SM_F32_VPL_MAX
#define ATTN_CFG_SM_F32_VPL_MAX 16
#endif
#ifndef ATTN_CFG_SM_H_VPL_MAX
#define ATTN_CFG_SM_H_VPL_MAX 32
#endif
static_assert(ATTN_CFG_SM_F32_VPL_MAX == 16 || ATTN_CFG_SM_F32_VPL_MAX == 32 ||
                  ATTN_CFG_SM_F32_VPL_MAX == 64, "fp32 values per lane");
static_assert(ATTN_CFG_SM_H_VPL_MAX == 16 || ATTN_CFG_SM_H_VPL_MAX == 32 ||
                  ATTN_CFG_SM_H_VPL_MAX == 64, "16-bit values per lane");
// 16-bit rows with 16-byte pieces keep the row in registers as loaded
// (packed, half the registers of fp32 values) and take each exponential
// twice, once for the sum and once for the output (1), or keep the
// exponentials as fp32 (0). Both give the same bits; the packed form
// measured 2-9% slower at 512 to 65536 columns (the second exponential and
// the unpacking cost more than the registers it frees), so 0 ships.
#ifndef ATTN_CFG_SM_PACKED
#define ATTN_CFG_SM_PACKED 0
#endif
template <typename V>
__device__ __forceinline__ V load_once(const V *p) {
  if (ATTN_CFG_SM_NONTEMPORAL) return __builtin_nontemporal_load(p);
  return *p;
}
template <typename V>
__device__ __forceinline__ void store_once(V v, V *p) {
  if (ATTN_CFG_SM_NONTEMPORAL) __builtin_nontemporal_store(v, p); else *p = v;
}

// Rows held in registers: VPL values per lane, WPR waves per row (64 * WPR
// lanes), N <= 64 * WPR * VPL. VEC: each lane moves 16-byte pieces (CH
// values), piece k of lane t at columns (k * 64 * WPR + t) * CH; otherwise
// value k of lane t is column k * 64 * WPR + t.
template <typename TIN, typename TOUT, int WPR, int VPL, bool VEC>
__global__ __launch_bounds__(rows_threads<WPR>()) void softmax_rows(SmParams p) {
  constexpr int ROWS = rows_threads<WPR>() / (64 * WPR);  // rows per workgroup
  constexpr int T = 64 * WPR;    // lanes per row
  constexpr int CH = 16 / sizeof(TIN);
  constexpr int NP = VEC ? VPL / CH : 0;  // 16-byte pieces per lane
  static_assert(!VEC || NP * CH == VPL, "whole pieces");
  __shared__ float red[16];
  const int wave = threadIdx.x >> 6;
  const int sub = wave / WPR;               // row of this workgroup
  const int t = threadIdx.x - sub * T;      // lane within the row
  const int64_t row = (int64_t)blockIdx.x * ROWS + sub;
  const bool live = row < p.M;              // uniform per wave
  const int N = p.N;
  const TIN *xr = static_cast<const TIN *>(p.x) + (live ? row : 0) * p.xs;
  TOUT *yr = static_cast<TOUT *>(p.y) + (live ? row : 0) * p.ys;

  if constexpr (ATTN_CFG_SM_PACKED && VEC && sizeof(TIN) == 2) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int OCH = 16 / sizeof(TOUT);  // output values per 16 bytes
    static_assert(CH % OCH == 0, "input piece covers whole output pieces");
    union Piece { u32x4 w; TIN e[CH]; };
    Piece raw[NP];  // piece k of this lane: columns (k * T + t) * CH ..
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int c0 = (k * T + t) * CH;
      raw[k].w = live && c0 < N ? load_once(reinterpret_cast<const u32x4 *>(xr + c0))
                                : u32x4{0, 0, 0, 0};
    }
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < NP; ++k)
      if ((k * T + t) * CH < N)
#pragma unroll
        for (int e = 0; e < CH; ++e) m = fmaxf(m, to_f32<TIN>(raw[k].e[e]));
    m = row_reduce<WPR, true>(m, red, wave) * kLog2e;
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < NP; ++k)
      if ((k * T + t) * CH < N)
#pragma unroll
        for (int e = 0; e < CH; ++e)
          l += __builtin_amdgcn_exp2f(fmaf(to_f32<TIN>(raw[k].e[e]), kLog2e, -m));
    l = row_reduce<WPR, false>(l, red, wave);
    const float inv = 1.0f / l;
    if (!live) return;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int c0 = (k * T + t) * CH;
      if (c0 >= N) continue;
#pragma unroll
      for (int s = 0; s < CH / OCH; ++s) {
        union { u32x4 w; TOUT e[OCH]; } u;
#pragma unroll
        for (int e = 0; e < OCH; ++e) {
          const float x = to_f32<TIN>(raw[k].e[s * OCH + e]);
          u.e[e] = from_f32<TOUT>(__builtin_amdgcn_exp2f(fmaf(x, kLog2e, -m)) * inv);
        }
        store_once(u.w, reinterpret_cast<u32x4 *>(yr + c0 + s * OCH));
      }
    }
    return;
  }

  float v[VPL];
  if constexpr (VEC) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int c0 = (k * T + t) * CH;
      union { u32x4 w; TIN e[CH]; } u;
      u.w = live && c0 < N ? load_once(reinterpret_cast<const u32x4 *>(xr + c0)) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < CH; ++e) v[k * CH + e] = live && c0 < N ? to_f32<TIN>(u.e[e]) : -INFINITY;
    }
  } else {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int c = k * T + t;
      v[k] = live && c < N ? to_f32<TIN>(xr[c]) : -INFINITY;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < VPL; ++k) m = fmaxf(m, v[k]);
  m = row_reduce<WPR, true>(m, red, wave) * kLog2e;
  float l = 0.f;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    v[k] = __builtin_amdgcn_exp2f(fmaf(v[k], kLog2e, -m));  // exp(-inf) = 0 for padding
    l += v[k];
  }
  l = row_reduce<WPR, false>(l, red, wave);
  const float inv = 1.0f / l;
  if (!live) return;
  if constexpr (VEC) {
    constexpr int OCH = 16 / sizeof(TOUT);  // output values per 16 bytes
    static_assert(CH % OCH == 0, "input piece covers whole output pieces");
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int c0 = (k * T + t) * CH;
      if (c0 >= N) continue;
#pragma unroll
      for (int s = 0; s < CH / OCH; ++s) {
        union { u32x4 w; TOUT e[OCH]; } u;
#pragma unroll
        for (int e = 0; e < OCH; ++e) u.e[e] = from_f32<TOUT>(v[k * CH + s * OCH + e] * inv);
        store_once(u.w, reinterpret_cast<u32x4 *>(yr + c0 + s * OCH));
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int c = k * T + t;
      if (c < N) yr[c] = from_f32<TOUT>(v[k] * inv);
    }
  }
}

// Long rows: one workgroup per row, two passes. Pass 1 keeps a running
// maximum and a running sum per thread (rescaled when the maximum grows),
// pass 2 re-reads the row and writes the normalised values.
// One value into the running (maximum, sum) of pass 1, in log2 units.
__device__ __forceinline__ void online_add(float x, float &m, float &l) {
  if (x > m) {
    l = l * __builtin_amdgcn_exp2f(m - x) + 1.f;  // 0 * ... when m was -inf
    m = x;
  } else if (x != -INFINITY) {
    l += __builtin_amdgcn_exp2f(x - m);
  }
}

template <typename TIN, typename TOUT, bool VEC>
__global__ __launch_bounds__(1024) void softmax_long(SmParams p) {
  constexpr int TH = 1024, CH = 16 / sizeof(TIN), OCH = 16 / sizeof(TOUT);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __shared__ float red[16];
  const int wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const int N = p.N;
  const TIN *xr = static_cast<const TIN *>(p.x) + row * p.xs;
  TOUT *yr = static_cast<TOUT *>(p.y) + row * p.ys;
  float m = -INFINITY, l = 0.f;
  if constexpr (VEC) {
    for (int c0 = threadIdx.x * CH; c0 < N; c0 += TH * CH) {
      union { u32x4 w; TIN e[CH]; } u;
      u.w = *reinterpret_cast<const u32x4 *>(xr + c0);
#pragma unroll
      for (int e = 0; e < CH; ++e) online_add(to_f32<TIN>(u.e[e]) * kLog2e, m, l);
    }
  } else {
    for (int c = threadIdx.x; c < N; c += TH) online_add(to_f32<TIN>(xr[c]) * kLog2e, m, l);
  }
  const float mr = row_reduce<16, true>(m, red, wave);
  l = l * (m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mr));
  const float inv = 1.0f / row_reduce<16, false>(l, red, wave);
  if constexpr (VEC) {
    for (int c0 = threadIdx.x * CH; c0 < N; c0 += TH * CH) {
      union { u32x4 w; TIN e[CH]; } u;
      u.w = *reinterpret_cast<const u32x4 *>(xr + c0);
#pragma unroll
      for (int s = 0; s < CH / OCH; ++s) {
        union { u32x4 w; TOUT e[OCH]; } o;
#pragma unroll
        for (int e = 0; e < OCH; ++e)
          o.e[e] = from_f32<TOUT>(
              __builtin_amdgcn_exp2f(fmaf(to_f32<TIN>(u.e[s * OCH + e]), kLog2e, -mr)) * inv);
        *reinterpret_cast<u32x4 *>(yr + c0 + s * OCH) = o.w;
      }
    }
  } else {
    for (int c = threadIdx.x; c < N; c += TH)
      yr[c] = from_f32<TOUT>(__builtin_amdgcn_exp2f(fmaf(to_f32<TIN>(xr[c]), kLog2e, -mr)) * inv);
  }
}

typedef void (*SmFn)(SmParams);

// 64 values per lane at 16 waves fit the 1024-thread register budget only
// with 16-byte loads; element loads stop at 32 (the host sends longer rows
// to the two-pass kernel).
template <typename TIN, typename TOUT, int WPR, bool VEC>
SmFn pick_vpl(int vpl) {
  constexpr int VMAX = (WPR == 16 && !VEC) ? 32 : 64;
  switch (vpl) {
    case 8: return softmax_rows<TIN, TOUT, WPR, 8, VEC>;
    case 16: return softmax_rows<TIN, TOUT, WPR, 16, VEC>;
    case 32: return softmax_rows<TIN, TOUT, WPR, 32, VEC>;
    default: return softmax_rows<TIN, TOUT, WPR, VMAX, VEC>;
  }
}

template <typename TIN, typename TOUT>
SmFn pick_kernel(int wpr, int vpl, bool vec, bool longrow) {
  if (longrow) return vec ? softmax_long<TIN, TOUT, true> : softmax_long<TIN, TOUT, false>;
  if (wpr == 1) return vec ? pick_vpl<TIN, TOUT, 1, true>(vpl) : pick_vpl<TIN, TOUT, 1, false>(vpl);
  if (wpr == 4) return vec ? pick_vpl<TIN, TOUT, 4, true>(vpl) : pick_vpl<TIN, TOUT, 4, false>(vpl);
  return vec ? pick_vpl<TIN, TOUT, 16, true>(vpl) : pick_vpl<TIN, TOUT, 16, false>(vpl);
}

SmFn pick(attn_dtype in, attn_dtype out, int wpr, int vpl, bool vec, bool longrow) {
  if (in == ATTN_F32) return pick_kernel<float, float>(wpr, vpl, vec, longrow);
  if (in == ATTN_BF16)
    return out == ATTN_F32 ? pick_kernel<__bf16, float>(wpr, vpl, vec, longrow)
                           : pick_kernel<__bf16, __bf16>(wpr, vpl, vec, longrow);
  return out == ATTN_F32 ? pick_kernel<_Float16, float>(wpr, vpl, vec, longrow)
                         : pick_kernel<_Float16, _Float16>(wpr, vpl, vec, longrow);
}

int esize(attn_dtype t) { return t == ATTN_F32 ? 4 : 2; }

}  // namespace

extern "C" {

attn_status attn_row_softmax(const void *x, int64_t x_row_stride, void *y, int64_t y_row_stride,
                             int64_t M, int64_t N, attn_dtype in_dtype, attn_dtype out_dtype,
                             void *stream) {
  if (!x || !y) return ATTN_ERR_NULL;
  if (M < 1 || N < 1 || M > INT32_MAX || N > (int64_t(1) << 30)) return ATTN_ERR_SHAPE;
  if (x_row_stride < N || y_row_stride < N || x_row_stride > (int64_t(1) << 40) ||
      y_row_stride > (int64_t(1) << 40))
    return ATTN_ERR_SHAPE;
  const bool in_ok = in_dtype == ATTN_F32 || in_dtype == ATTN_F16 || in_dtype == ATTN_BF16;
  if (!in_ok) return ATTN_ERR_UNSUPPORTED;
  if (out_dtype != in_dtype && out_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  const int ei = esize(in_dtype), eo = esize(out_dtype);
  if ((reinterpret_cast<uintptr_t>(x) % ei) != 0 || (reinterpret_cast<uintptr_t>(y) % eo) != 0)
    return ATTN_ERR_UNSUPPORTED;
  // 16-byte pieces when every row starts 16-byte aligned and N is whole pieces
  const int ch = 16 / ei;
  const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(y) & 15) == 0 && (x_row_stride * ei) % 16 == 0 &&
                   (y_row_stride * eo) % 16 == 0 && N % ch == 0;
  int wpr = 1, vpl = 8;
  bool longrow = false;
  const int64_t v14 = ei == 4 ? ATTN_CFG_SM_F32_VPL_MAX : ATTN_CFG_SM_H_VPL_MAX;  // 1 or 4 waves
  if (N <= 64 * v14) {
    wpr = 1;
  } else if (N <= 256 * v14) {
    wpr = 4;
  } else if (N <= 1024 * (vec ? 64 : 32)) {
    wpr = 16;
  } else {
    longrow = true;
  }
  if (!longrow) {
    const int64_t lanes = 64 * wpr;
    while ((int64_t)vpl * lanes < N) vpl *= 2;
  }
  SmParams p;
  p.x = x;
  p.y = y;
  p.xs = x_row_stride;
  p.ys = y_row_stride;
  p.M = (int)M;
  p.N = (int)N;
  const int64_t rows_per_wg = longrow || wpr > 1 ? 1 : 4;
  const int threads = longrow ? 1024 : wpr == 1 ? 256 : 64 * wpr;
  const int64_t grid = (M + rows_per_wg - 1) / rows_per_wg;
  SmFn fn = pick(in_dtype, out_dtype, wpr, vpl, vec, longrow);
  void *args[] = {&p};
  const hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((unsigned)grid),
                                         dim3(threads), args, 0, (hipStream_t)stream);
  if (err != hipSuccess) {
    attn_internal::set_last_hip_error((int)err);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // extern "C"
