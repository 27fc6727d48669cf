// General-layout attention forward for gfx950 (MI355X): the same operation
// as attn_fwd (entry point attn_fwd_strided), for
//  - a different number of keys than queries (cross-attention;
//    "Programming an attention kernel in Triton", section "Kernel 4:
//    bringing it together, a self-attention kernel", checks its kernel on
//    mismatched query and key lengths);
//  - head dimensions d <= 128 other than 64 and 128, multiple of 8, computed
//    at D = 64 or 128 with the extra columns read as zeros (the padding note
//    of "4.4 Writing GPU Kernels with Triton", section "Sizing the attention
//    kernel"). This changes nothing: a zero column contributes 0 to every
//    dot product q.k, and the output columns past d are never written;
//  - strided tensors: element (b, h, n, c) at b*sb + h*sh + n*sn + c (the
//    Triton kernels of the same pages take per-dimension strides).
// bf16/fp16 problems with row strides of at most 2^21 elements run on
// attn_fwd's tuned kernels, whose strided instances cover all three cases
// (fwd16_strided); the kernels below serve fp32 inputs and longer row
// strides, and every problem when built with ATTN_CFG_STRIDED_TUNED=0.
//
// attn_gen_16 (bf16 / fp16): one workgroup per (head, 128 queries); 4 waves
// of 32 queries each loop over 64-key tiles. Per 32-key block and wave:
// S^T = K Q^T on v_mfma_f32_32x32x16 (Q in registers), mask, online softmax
// (running maximum with a lazy rescale, running sum), P packed to fp16, and
// O^T += V^T P^T on the fp16 matrix core; for bf16 inputs V is converted to
// fp16 in LDS, as attn_fwd does. K and V tiles stream through a two-stage
// LDS ring filled by buffer_load ... lds; each lane's source offset follows
// the row stride, and its 16-byte piece is fetched from an out-of-range
// offset (read as zeros) when it lies past column d.
// attn_gen_f32 (fp32): the same decomposition with plain loads and the fp32
// matrix core (v_mfma_f32_32x32x2_f32).

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"
#include "mfma_pipe.h"

namespace attn_internal {
void set_last_hip_error(int e);
// The tuned bf16/fp16 forward (attn_fwd.hip) on strided tensors: whether it
// takes a problem, and its launch.
bool fwd16_takes_strided(int64_t Nk, int64_t d, attn_dtype in_dtype, const int64_t *st);
attn_status fwd16_strided(const void *q, const void *k, const void *v, void *o, float *lse,
                          int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                          float scale, attn_dtype in_dtype, attn_dtype out_dtype, void *stream,
                          const int64_t *st);
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kBlockM = 128;   // queries per workgroup (32 per wave)
// Keys per step (bf16 / fp16), per head dimension: the sweep of this choice
// (io_aware_attention_flash_amd/sweep.py) measured 32 fastest at d = 128 and
// 64 at d = 64. -D ATTN_CFG_GEN_TILE_K overrides both.
template <int D>
constexpr int gen_tile_k() {
#ifdef ATTN_CFG_GEN_TILE_K
  return ATTN_CFG_GEN_TILE_K;
#else
  return D == 128 ? 32 : 64;
#endif
}
static_assert(gen_tile_k<64>() % 32 == 0 && gen_tile_k<64>() <= 128 && gen_tile_k<128>() % 32 == 0 &&
                  gen_tile_k<128>() <= 128, "key tile");
constexpr int kTileKMax = 128;  // the largest key tile any build uses
#ifndef ATTN_CFG_GEN_LOOKAHEAD  // MFMA steps by which LDS operand reads run ahead
#define ATTN_CFG_GEN_LOOKAHEAD 2
#endif
constexpr int kGenLookahead = ATTN_CFG_GEN_LOOKAHEAD;
static_assert(kGenLookahead >= 1 && kGenLookahead <= 4, "lookahead range");
constexpr float kRescaleLog2 = 8.0f;
// Strided bf16/fp16 problems on the tuned kernels (1) or on this file's
// kernel (0).
#ifndef ATTN_CFG_STRIDED_TUNED
#define ATTN_CFG_STRIDED_TUNED 1
#endif
// Stores of O with the non-temporal hint or plain. Each lane stores 16-byte
// pieces of its own row, not whole lines, and the hint measured 3-5% slower:
// plain.
#ifndef ATTN_CFG_GEN_O_NONTEMPORAL
#define ATTN_CFG_GEN_O_NONTEMPORAL 0
#endif

template <class T>
__device__ __forceinline__ void store_o(T *dst, const T &val) {
  if (ATTN_CFG_GEN_O_NONTEMPORAL) __builtin_nontemporal_store(val, dst); else *dst = val;
}
constexpr uint32_t kOutOfRange = 0x80000000u;  // a source offset past any range

struct GenParams {
  const void *q, *k, *v;
  void *o;
  float *lse;               // [B][H][Nq] contiguous
  int64_t qs[3], ks[3], vs[3], os[3];  // element strides of b, h, n
  int H, BH, Nq, Nk, d, nq;
  float qk;                 // scale * log2(e), >= FLT_MIN
};

// ---------------------------------------------------------------- helpers

template <int D>
__device__ __forceinline__ int swz(int row) {  // see attn_bwd.hip: row and transposing reads
  if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  const int r = (row >> 1) & 7;
  return ((r & 3) << 1) | (r >> 2);
}

template <int D>
__device__ __forceinline__ u32x4 row_frag(const uint16_t *tile, int row, int chunk) {
  return *reinterpret_cast<const u32x4 *>(tile + row * D + ((chunk ^ swz<D>(row)) << 3));
}

template <int D>
struct TrAddr {
  int off[D / 32][2];
};

template <int D>
__device__ __forceinline__ TrAddr<D> tr_addr(int lane) {
  TrAddr<D> ta;
  const int g = lane >> 5, h = (lane >> 4) & 1, s = lane & 15;
  const int a = s & 3, m = s >> 2;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 8 * u + 4 * g + m;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const int x = 4 * cb + 2 * h + (a >> 1);
      ta.off[cb][u] = row * D + ((x ^ swz<D>(row)) << 3) + (a & 1) * 4;
    }
  }
  return ta;
}

// Operand contracting over rows 16t .. 16t+15 of a row-major tile: lane l
// gets column 32cb + (l & 31) at rows 16t + 4g + 0..3 and 16t + 8 + 4g + 0..3.
template <int D>
__device__ __forceinline__ u32x4 tr_frag(const uint16_t *tile, const TrAddr<D> &ta, int t, int cb) {
  const uint16_t *p = tile + 16 * t * D;
  const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p + ta.off[cb][0]));
  const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p + ta.off[cb][1]));
  const u32x2 w0 = __builtin_bit_cast(u32x2, r0), w1 = __builtin_bit_cast(u32x2, r1);
  return u32x4{w0[0], w0[1], w1[0], w1[1]};
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

template <bool IS_BF16>
__device__ __forceinline__ f32x16 mfma_in(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (IS_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ u32x4 make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xFFFFu,
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), (uint32_t)kBufferFlags};
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// 16 bytes per lane from the descriptor's range (reads past it give zeros)
// into LDS at M0 + 16 * lane (see attn_fwd.hip for why this is inline asm).
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds_byte, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_byte), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ------------------------------------------------ strided tile copies

// R rows x D columns (16-bit) of a strided matrix into a swizzled LDS tile:
// instruction c fills slots c*256 + tid; slot s holds physical chunk
// s % CPR of row s / CPR, i.e. logical chunk (s % CPR) ^ swz(row). The lane
// reads row (c * RPI + tid / CPR) of the source at stride sn, or nothing
// (zeros) when its logical chunk starts at or past column d.
template <int D, int R>
struct GenCopy {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = kThreads / CPR;  // rows per instruction
  static constexpr int INS = R / RPI;
  static_assert(INS * RPI == R && RPI % 16 == 0, "copy shape");
  uint32_t off0;  // source byte offset of instruction 0, or kOutOfRange
  uint32_t step;  // bytes between instructions: RPI rows
  __device__ void init(int tid, int64_t sn, int d) {
    const int row = tid / CPR, lc = (tid % CPR) ^ swz<D>(row);
    off0 = lc * 8 < d ? (uint32_t)(row * sn * 2 + lc * 16) : kOutOfRange;
    step = (uint32_t)(RPI * sn * 2);
  }
  // rows [r0, min(r0 + R, n)) of the matrix at `base` (rows of stride sn).
  __device__ void issue(const uint16_t *base, int64_t sn, int r0, int n, int d, uint16_t *lds,
                        int wave) const {
    const int rows = min(n - r0, R);
    const uint32_t bytes = rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * sn + d) * 2) : 0u;
    const u32x4 rs = make_rsrc(base + (rows > 0 ? (int64_t)r0 * sn : 0), bytes);
    const uint32_t ldsb = __builtin_amdgcn_readfirstlane(lds_addr(lds) + wave * 64 * 16);
#pragma unroll
    for (int c = 0; c < INS; ++c)
      dma16(rs, ldsb + c * kThreads * 16, off0 == kOutOfRange ? kOutOfRange : off0 + c * step);
  }
};

// ------------------------------------------ bf16 V beyond fp16's range

// The P.V product runs on fp16 copies of bf16 V, so a value with
// |v| > 65504 became +-inf there and the accumulators of every wave that met
// it are not finite. Such a wave recomputes its rows' outputs the way the
// page's kernel does: P rounded to bf16, V as given, bf16 x bf16 on the
// matrix cores with fp32 accumulation, K and V read straight from memory
// (strided, columns past d as zeros), against the final reference maximum m
// (every score is within 2^8 of it, so every weight is <= 2^8). Returns this
// lane's sum of the bf16-rounded weights; acc is overwritten.
template <int D, bool CAUSAL>
__device__ __forceinline__ float redo_rows_bf16(const GenParams &p, const uint16_t *Kh,
                                                const uint16_t *Vh, int qw0, int qrow, int g,
                                                int l32, const u32x4 *qf, float m,
                                                f32x16 (&acc)[D / 32]) {
  constexpr int NKC = D / 16, NCB = D / 32;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const int Nk = p.Nk, d = p.d;
  const int64_t ks = p.ks[2], vs = p.vs[2];
  const int kend = CAUSAL ? min(Nk, qw0 + 32) : Nk;
  const float qk = p.qk, mref = m == -INFINITY ? 0.f : m;
  float l = 0.f;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
#pragma unroll 1
  for (int k0 = 0; k0 < kend; k0 += 32) {
    const int key = k0 + l32;
    const uint16_t *krow = Kh + (int64_t)(key < Nk ? key : 0) * ks + 8 * g;
    f32x16 sc = f32x16{};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      u32x4 kf = u32x4{0, 0, 0, 0};
      if (key < Nk && 16 * kc + 8 * g < d) kf = *reinterpret_cast<const u32x4 *>(krow + 16 * kc);
      sc = mfma_in<true>(kf, qf[kc], sc);
    }
    uint32_t pb[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      float w[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int kk = k0 + 8 * ((e + i) >> 2) + 4 * g + ((e + i) & 3);
        const bool dead = kk >= Nk || (CAUSAL && kk > qrow);
        w[i] = dead ? 0.f : __builtin_amdgcn_exp2f(sc[e + i] * qk - mref);
      }
      const bf16x2 hh = {(__bf16)w[0], (__bf16)w[1]};
      l += (float)hh[0] + (float)hh[1];
      pb[e >> 1] = __builtin_bit_cast(uint32_t, hh);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pf = {pb[4 * t], pb[4 * t + 1], pb[4 * t + 2], pb[4 * t + 3]};
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int col = 32 * cb + l32;
        uint32_t vv[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int kk = k0 + 16 * t + 8 * (x >> 2) + 4 * g + (x & 3);
          vv[x] = kk < Nk && col < d ? Vh[(int64_t)kk * vs + col] : 0u;
        }
        const u32x4 a = {vv[0] | (vv[1] << 16), vv[2] | (vv[3] << 16), vv[4] | (vv[5] << 16),
                         vv[6] | (vv[7] << 16)};
        acc[cb] = mfma_in<true>(a, pf, acc[cb]);
      }
    }
  }
  return l;
}

// ------------------------------------------------- bf16 / fp16 kernel

template <int D, int TK_ = gen_tile_k<D>()>
struct GenShape {
  static constexpr int TK = TK_;
  static constexpr int TILE = TK * D;
  static constexpr int STAGE = 2 * TILE;  // K, V
  static constexpr int LDS_ELEMS = 2 * STAGE;
};

template <int D, bool IS_BF16, bool CAUSAL, bool OUT_F32, int TK = gen_tile_k<D>()>
__global__ __launch_bounds__(kThreads, 2) void attn_gen_16(GenParams p) {
  using S = GenShape<D, TK>;
  constexpr int kTileK = S::TK;
  using Copy = GenCopy<D, kTileK>;
  constexpr int NKC = D / 16, NCB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::LDS_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int t_ = blockIdx.x / p.BH, bh = blockIdx.x - t_ * p.BH;
  const int b = bh / p.H, h = bh - b * p.H;
  const int qt = CAUSAL ? p.nq - 1 - t_ : t_;  // causal: longest first
  const int Nq = p.Nq, Nk = p.Nk, d = p.d;
  const int m0 = qt * kBlockM, qw0 = m0 + 32 * wave, qrow = qw0 + l32;
  const uint16_t *Qh = static_cast<const uint16_t *>(p.q) + b * p.qs[0] + h * p.qs[1];
  const uint16_t *Kh = static_cast<const uint16_t *>(p.k) + b * p.ks[0] + h * p.ks[1];
  const uint16_t *Vh = static_cast<const uint16_t *>(p.v) + b * p.vs[0] + h * p.vs[1];

  Copy kc_, vc_;
  kc_.init(tid, p.ks[2], d);
  vc_.init(tid, p.vs[2], d);
  const int kend = CAUSAL ? min(Nk, m0 + kBlockM) : Nk;
  const int n_kt = (kend + kTileK - 1) / kTileK;
  auto stage = [&](int s) { return lds + s * S::STAGE; };
  auto issue = [&](int it) {
    uint16_t *st = stage(it & 1);
    kc_.issue(Kh, p.ks[2], it * kTileK, Nk, d, st, wave);
    vc_.issue(Vh, p.vs[2], it * kTileK, Nk, d, st + S::TILE, wave);
  };
  // bf16 V: this thread's own 16-byte slots of the V tile, to fp16 in place
  // once its copies have landed.
  auto convert_v = [&](int it) {
    if constexpr (IS_BF16) {
      uint16_t *vt = stage(it & 1) + S::TILE;
#pragma unroll
      for (int c = 0; c < Copy::INS; ++c) {
        u32x4 *slot = reinterpret_cast<u32x4 *>(vt + (c * kThreads + tid) * 8);
        const u32x4 x = *slot;
        u32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = pack_f16(bf16_lo(x[e]), bf16_hi(x[e]));
        *slot = y;
      }
    }
  };
  issue(0);

  // Q operand of S^T = K Q^T: Q[qrow][16kc + 8g .. +7], zeros past d or Nq.
  u32x4 qf[NKC];
  {
    const bool ok = qrow < Nq;
    const uint16_t *qr = Qh + (int64_t)(ok ? qrow : 0) * p.qs[2];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int c0 = 16 * kc + 8 * g;
      qf[kc] = ok && c0 < d ? *reinterpret_cast<const u32x4 *>(qr + c0) : u32x4{0, 0, 0, 0};
    }
  }
  const TrAddr<D> ta = tr_addr<D>(lane);
  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float qk = p.qk;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

#pragma unroll 1
  for (int it = 0; it < n_kt; ++it) {
    if (it + 1 < n_kt) {
      issue(it + 1);
      wait_vmcnt<2 * Copy::INS>();
    } else {
      wait_vmcnt<0>();
    }
    convert_v(it);
    lds_barrier();
    const uint16_t *kt = stage(it & 1), *vt = kt + S::TILE;
#pragma unroll
    for (int kb = 0; kb < kTileK / 32; ++kb) {
      const int key0 = it * kTileK + 32 * kb;
      if (CAUSAL && key0 > qw0 + 31) continue;  // every key after every query of this wave
      if (key0 >= Nk) continue;
      // S^T: lane (query qrow) holds keys key0 + 8j + 4g + r in s[4j + r].
      f32x16 s = f32x16{};
      mfma_pipelined<NKC, kGenLookahead>(
          [&](int kc) { return row_frag<D>(kt, 32 * kb + l32, 2 * kc + g); },
          [&](int kc, const u32x4 &a) { s = mfma_in<IS_BF16>(a, qf[kc], s); });
      // Masked pairs only on the diagonal or past the last key: one
      // wave-uniform branch around all 16 selects.
      if ((CAUSAL && key0 + 31 > qw0) || key0 + 32 > Nk) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + 8 * (e >> 2) + 4 * g + (e & 3);
          const bool keep = (!CAUSAL || key <= qrow) && key < Nk;
          s[e] = keep ? s[e] : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * qk;  // both key halves of this query
      // Lazy rescale: the state moves to a new maximum only when it grew by
      // more than 2^8 (every p stays <= 256, which fp16 holds exactly enough);
      // the same reference serves the output and the sum.
      if (__any(mx > m + kRescaleLog2)) {
        const float mn = fmaxf(m, mx);
        // 0 when m was -inf; 1 for a lane with no visible key yet (state all 0)
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
        l *= alpha;
        m = mn;
      }
      const float mref = m == -INFINITY ? 0.f : m;
      uint32_t pp[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[e] * qk - mref);
        const float p1 = __builtin_amdgcn_exp2f(s[e + 1] * qk - mref);
        pp[e >> 1] = pack_f16(p0, p1);
        // the row sum takes the rounded weights, as the products do: one
        // fp16 pair dot (1, 1) accumulated in fp32
        l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pp[e >> 1]), ones, l, false);
      }
      // O^T += V^T P^T
      mfma_pipelined<2 * NCB, kGenLookahead>(  // step i: t = i / NCB, cb = i % NCB
          [&](int i) { return tr_frag<D>(vt + 32 * kb * D, ta, i / NCB, i % NCB); },
          [&](int i, const u32x4 &a) {
            const int t = i / NCB;
            const u32x4 pf = {pp[4 * t], pp[4 * t + 1], pp[4 * t + 2], pp[4 * t + 3]};
            acc[i % NCB] = mfma_f16(a, pf, acc[i % NCB]);
          });
    }
    lds_barrier();
  }

  const float l_tot = l + __shfl_xor(l, 32);
  const float l_safe = l_tot > 0.f ? l_tot : 1.f;
  float inv = 1.0f / l_safe;
  // bf16 V with |v| > 65504 became +-inf in its fp16 copy: recompute this
  // wave's outputs with bf16 P against the given V (see redo_rows_bf16).
  if (IS_BF16) {
    bool bad = false;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) bad |= !__builtin_isfinite(acc[cb][r]);
    if (__any(bad)) {
      const float lb = redo_rows_bf16<D, CAUSAL>(p, Kh, Vh, qw0, qrow, g, l32, qf, m, acc);
      const float lt = lb + __shfl_xor(lb, 32);
      inv = 1.0f / (lt > 0.f ? lt : 1.f);
    }
  }
  if (qrow < Nq) {
    if (g == 0)
      p.lse[(size_t)bh * Nq + qrow] =
          (m == -INFINITY ? -INFINITY : (m + __builtin_amdgcn_logf(l_safe)) * 0.69314718055994531f);
    uint8_t *orow = static_cast<uint8_t *>(p.o) +
                    (b * p.os[0] + h * p.os[1] + (int64_t)qrow * p.os[2]) * (OUT_F32 ? 4 : 2);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c0 = 32 * cb + 8 * j + 4 * g;
        if (c0 >= d) continue;
        const float o0 = acc[cb][4 * j] * inv, o1 = acc[cb][4 * j + 1] * inv;
        const float o2 = acc[cb][4 * j + 2] * inv, o3 = acc[cb][4 * j + 3] * inv;
        if constexpr (OUT_F32) {
          store_o(reinterpret_cast<f32x4 *>(orow + c0 * 4), f32x4{o0, o1, o2, o3});
        } else if constexpr (IS_BF16) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          store_o(reinterpret_cast<bf16x4 *>(orow + c0 * 2),
                  bf16x4{(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3});
        } else {
          typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
          store_o(reinterpret_cast<f16x4 *>(orow + c0 * 2),
                  f16x4{(_Float16)o0, (_Float16)o1, (_Float16)o2, (_Float16)o3});
        }
      }
  }
}

// ---------------------------------------------------------- fp32 kernel

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_gen_f32(GenParams p) {
  constexpr int BN = 32;
  constexpr int KSTR = D + 2, VSTR = D + 8;  // conflict-free column reads
  constexpr int NCB = D / 32;
  __shared__ float lk[BN * KSTR];
  __shared__ float lv[BN * VSTR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int t_ = blockIdx.x / p.BH, bh = blockIdx.x - t_ * p.BH;
  const int b = bh / p.H, h = bh - b * p.H;
  const int qt = CAUSAL ? p.nq - 1 - t_ : t_;
  const int Nq = p.Nq, Nk = p.Nk, d = p.d;
  const int m0 = qt * kBlockM;
  const float *Qh = static_cast<const float *>(p.q) + b * p.qs[0] + h * p.qs[1];
  const float *Kh = static_cast<const float *>(p.k) + b * p.ks[0] + h * p.ks[1];
  const float *Vh = static_cast<const float *>(p.v) + b * p.vs[0] + h * p.vs[1];

  const int qrow = m0 + wave * 32 + l32;
  float qf[D / 2];  // Q[qrow][2kk + g]
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) {
    const int c = 2 * kk + g;
    qf[kk] = qrow < Nq && c < d ? Qh[(int64_t)qrow * p.qs[2] + c] : 0.f;
  }
  const int kend = CAUSAL ? min(Nk, m0 + kBlockM) : Nk;
  const int n_tiles = (kend + BN - 1) / BN;

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
  float m_i = -INFINITY, l_i = 0.f;
  const float qk = p.qk;

  for (int j = 0; j < n_tiles; ++j) {
    const int n0 = j * BN;
    __syncthreads();  // previous tile fully consumed
    for (int e = tid; e < BN * D; e += kThreads) {
      const int row = e / D, col = e % D;
      const int key = n0 + row;
      const bool ok = key < Nk && col < d;
      lk[row * KSTR + col] = ok ? Kh[(int64_t)key * p.ks[2] + col] : 0.f;
      lv[row * VSTR + col] = ok ? Vh[(int64_t)key * p.vs[2] + col] : 0.f;
    }
    __syncthreads();
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(lk[l32 * KSTR + 2 * kk + g], qf[kk], s, 0, 0, 0);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = n0 + 8 * (r >> 2) + 4 * g + (r & 3);
      const bool dead = key >= Nk || (CAUSAL && key > qrow);
      s[r] = dead ? -INFINITY : s[r];
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx * qk);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_i - m_use);
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], qk, -m_use));
      lsum += s[r];
    }
    l_i = l_i * alpha + lsum;
    m_i = m_new;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * g + (r & 3);
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(lv[key * VSTR + cb * 32 + l32], s[r],
                                                       acc[cb], 0, 0, 0);
      }
    }
  }

  const float l_tot = l_i + __shfl_xor(l_i, 32);
  const float l_safe = l_tot > 0.f ? l_tot : 1.f;
  const float inv = 1.0f / l_safe;
  if (qrow < Nq) {
    if (g == 0)
      p.lse[(size_t)bh * Nq + qrow] =
          (m_i == -INFINITY ? -INFINITY : (m_i + __builtin_amdgcn_logf(l_safe)) * 0.69314718055994531f);
    float *orow = static_cast<float *>(p.o) + b * p.os[0] + h * p.os[1] + (int64_t)qrow * p.os[2];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c0 = cb * 32 + r4 * 8 + g * 4;
        if (c0 >= d) continue;
        *reinterpret_cast<f32x4 *>(orow + c0) =
            f32x4{acc[cb][4 * r4] * inv, acc[cb][4 * r4 + 1] * inv, acc[cb][4 * r4 + 2] * inv,
                  acc[cb][4 * r4 + 3] * inv};
      }
  }
}

// ------------------------------------------------------------------ host

typedef void (*GenFn)(GenParams);

template <int D, bool IS_BF16, int TK>
GenFn pick16_tk(bool causal, bool out_f32) {
  if (causal)
    return out_f32 ? attn_gen_16<D, IS_BF16, true, true, TK> : attn_gen_16<D, IS_BF16, true, false, TK>;
  return out_f32 ? attn_gen_16<D, IS_BF16, false, true, TK> : attn_gen_16<D, IS_BF16, false, false, TK>;
}

// At d = 64, short key sequences take 128-key tiles: half the iterations, so
// half the per-iteration copies and barriers, which dominate a short loop;
// for long ones the larger LDS stages cost occupancy. Measured: +8.8% at
// 1024 keys, -8.5% at 3000. Outputs are the same bits either way (the 32-key
// blocks run in the same order).
constexpr int64_t kGenShortKeys = 1024;

template <int D, bool IS_BF16>
GenFn pick16(bool causal, bool out_f32, int64_t Nk) {
#ifndef ATTN_CFG_GEN_TILE_K
  if constexpr (D == 64)
    if (Nk <= kGenShortKeys) return pick16_tk<D, IS_BF16, 128>(causal, out_f32);
#endif
  (void)Nk;
  return pick16_tk<D, IS_BF16, gen_tile_k<D>()>(causal, out_f32);
}

template <int D>
GenFn pick(attn_dtype in, bool causal, bool out_f32, int64_t Nk) {
  if (in == ATTN_F32) return causal ? attn_gen_f32<D, true> : attn_gen_f32<D, false>;
  if (in == ATTN_BF16) return pick16<D, true>(causal, out_f32, Nk);
  return pick16<D, false>(causal, out_f32, Nk);
}

int elem_bytes(attn_dtype t) { return t == ATTN_F32 ? 4 : 2; }

// Strides (elements) of a [B][H][n][d] view: the given ones, or contiguous.
void fill_strides(int64_t out[3], const int64_t *in, int64_t H, int64_t n, int64_t d) {
  if (in) {
    out[0] = in[0], out[1] = in[1], out[2] = in[2];
  } else {
    out[2] = d, out[1] = n * d, out[0] = H * n * d;
  }
}

// Every element (b, h, i, c) of the view has a non-negative offset below
// 2^47 elements, rows do not overlap (row stride >= d), and every row starts
// 16-byte aligned.
bool view_ok(const void *ptr, const int64_t s[3], int64_t B, int64_t H, int64_t n, int64_t d,
             int eb) {
  if (s[0] < 0 || s[1] < 0 || s[2] < d) return false;
  const int64_t lim = int64_t(1) << 47;
  if (s[0] > lim / B || s[1] > lim / H || s[2] > lim / n) return false;
  if ((reinterpret_cast<uintptr_t>(ptr) & 15) != 0) return false;
  for (int i = 0; i < 3; ++i)
    if ((s[i] * eb) % 16 != 0) return false;
  return true;
}

// Whether the B*H blocks of n rows x d elements of a view with (batch, head,
// row) strides s cover disjoint elements, so that no two output rows share
// memory (an expanded view, stride 0 over heads or batches, is refused).
// Ordered by stride, each dimension of extent > 1 must step past everything
// inside it; the row stride is already >= d.
bool out_view_disjoint(const int64_t s[3], int64_t B, int64_t H, int64_t n, int64_t d) {
  int64_t st[3] = {s[0], s[1], s[2]}, ext[3] = {B, H, n};
  for (int i = 0; i < 3; ++i)  // ascending stride
    for (int j = i + 1; j < 3; ++j)
      if (st[j] < st[i] || (st[j] == st[i] && ext[j] > ext[i])) {
        const int64_t a = st[i], b = ext[i];
        st[i] = st[j], ext[i] = ext[j], st[j] = a, ext[j] = b;
      }
  int64_t span = d;  // elements covered by the dimensions inside the current one
  for (int i = 0; i < 3; ++i) {
    if (ext[i] == 1) continue;
    if (st[i] < span) return false;
    span += (ext[i] - 1) * st[i];
  }
  return true;
}

}  // namespace

extern "C" {

attn_status attn_fwd_strided(const void *q, const int64_t *q_strides, const void *k,
                             const int64_t *k_strides, const void *v, const int64_t *v_strides,
                             void *o, const int64_t *o_strides, float *lse, int64_t B, int64_t H,
                             int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                             attn_dtype in_dtype, attn_dtype out_dtype, void *stream) {
  // Validation first: no HIP call happens before every argument is checked.
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_ERR_SHAPE;
  if (Nq > (int64_t(1) << 24) || Nk > (int64_t(1) << 24) || B * H > (int64_t(1) << 24))
    return ATTN_ERR_SHAPE;
  if (causal && Nq != Nk) return ATTN_ERR_SHAPE;
  if (d < 8 || d > 128 || d % 8 != 0) return ATTN_ERR_UNSUPPORTED;
  const bool in_ok = in_dtype == ATTN_F32 || in_dtype == ATTN_F16 || in_dtype == ATTN_BF16;
  if (!in_ok) return ATTN_ERR_UNSUPPORTED;
  if (in_dtype == ATTN_F32 && out_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (in_dtype != ATTN_F32 && out_dtype != in_dtype && out_dtype != ATTN_F32)
    return ATTN_ERR_UNSUPPORTED;
  if (!(scale >= 0.f) || !isfinite(scale)) return ATTN_ERR_SCALE;
  GenParams p;
  fill_strides(p.qs, q_strides, H, Nq, d);
  fill_strides(p.ks, k_strides, H, Nk, d);
  fill_strides(p.vs, v_strides, H, Nk, d);
  fill_strides(p.os, o_strides, H, Nq, d);
  const int eb = elem_bytes(in_dtype), ob = elem_bytes(out_dtype);
  if (!view_ok(q, p.qs, B, H, Nq, d, eb) || !view_ok(k, p.ks, B, H, Nk, d, eb) ||
      !view_ok(v, p.vs, B, H, Nk, d, eb) || !view_ok(o, p.os, B, H, Nq, d, ob) ||
      !out_view_disjoint(p.os, B, H, Nq, d))
    return ATTN_ERR_UNSUPPORTED;
  // a key tile (up to kTileKMax rows) of K or V must fit the 32-bit range of a buffer descriptor
  if (in_dtype != ATTN_F32 && (p.ks[2] * eb * kTileKMax >= (int64_t(1) << 31) ||
                               p.vs[2] * eb * kTileKMax >= (int64_t(1) << 31)))
    return ATTN_ERR_UNSUPPORTED;
  // bf16/fp16 runs on the tuned kernels, which read and write rows through
  // the same strides.
  if (ATTN_CFG_STRIDED_TUNED) {
    int64_t st[12];
    for (int i = 0; i < 3; ++i)
      st[i] = p.qs[i], st[3 + i] = p.ks[i], st[6 + i] = p.vs[i], st[9 + i] = p.os[i];
    if (attn_internal::fwd16_takes_strided(Nk, d, in_dtype, st))
      return attn_internal::fwd16_strided(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale,
                                          in_dtype, out_dtype, stream, st);
  }
  const int64_t nq = (Nq + kBlockM - 1) / kBlockM;
  const int64_t grid = nq * B * H;
  if (grid > INT32_MAX) return ATTN_ERR_SHAPE;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.H = (int)H;
  p.BH = (int)(B * H);
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.d = (int)d;
  p.nq = (int)nq;
  const double qk = (double)scale * 1.4426950408889634;
  p.qk = qk < (double)FLT_MIN ? FLT_MIN : (float)qk;
  const bool out_f32 = out_dtype == ATTN_F32;
  GenFn fn = d <= 64 ? pick<64>(in_dtype, causal != 0, out_f32, Nk)
                     : pick<128>(in_dtype, causal != 0, out_f32, Nk);
  void *args[] = {&p};
  const hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((unsigned)grid),
                                         dim3(kThreads), args, 0, (hipStream_t)stream);
  if (err != hipSuccess) {
    attn_internal::set_last_hip_error((int)err);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // extern "C"
