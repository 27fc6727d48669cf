// FlashAttention backward for gfx950 (MI355X): dQ, dK, dV of
// O = softmax(scale Q K^T [+ causal mask]) V from the upstream gradient dO,
// the forward's O and its per-row natural-log logsumexp L.
//
// The method is that of "4.4 Writing GPU Kernels with Triton", section
// "Kernel 5: FlashAttention Backward": the softmax weights are rebuilt tile by
// tile from L (P = exp(S - L), no N x N tensor in memory), D_i = rowsum(dO_i *
// O_i) collapses the softmax Jacobian, dS = P * (dP - D), dV = P^T dO,
// dK = scale dS^T Q and dQ = scale dS K. The page's closing notes describe
// the atomic-free split used here: a key-parallel kernel owns dK and dV, a
// query-parallel kernel owns dQ, and neither writes the other's rows, so
// there are no atomics and the result is deterministic.
//
// Two launches on the caller's stream for bf16/fp16 inputs (dQ first, then
// dK/dV), three for fp32 (bwd_prep, dK/dV, dQ):
//   bwd_prep : LD[row] = (L * log2(e), D) per query row, into the workspace;
//              for 16-bit inputs bwd_dq does this step for its own rows.
//   bwd_dkdv : one workgroup per (head, 128 keys); 4 waves of 32 keys each
//              loop over 32-query tiles. Per tile and wave, on the matrix
//              cores (v_mfma_f32_32x32x16, fp32 accumulate):
//                S = Q K^T, P = exp2(S*qk - L*log2 e), dV^T += dO^T P,
//                dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS.
//              K stays in registers, V in LDS; Q, dO and LD tiles stream
//              through a two-stage LDS ring filled by buffer_load ... lds.
//   bwd_dq   : one workgroup per (head, 128 queries); 4 waves of 32 queries
//              loop over 64-key tiles: S^T = K Q^T, P, dP^T = V dO^T,
//              dS, dQ^T += K^T dS^T. Q and dO stay in registers; K and V
//              tiles stream through a two-stage LDS ring. Its rows' D comes
//              from dO (already in registers) and O, read once.
// P and dS enter the matrix cores in the input type (bf16 or fp16), as the
// page casts them to the operand type; S, P, dP, dS and every accumulator
// are fp32. In both loops every MFMA's LDS operands are read a fixed number
// of steps ahead (mfma_pipe.h), the masking of edge tiles sits under one
// wave-uniform branch, and the register operands are loaded completely
// before the loop, so no wait inside it covers the tile copies in flight.

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "attn.h"
#include "mfma_pipe.h"

namespace attn_internal {
void set_last_hip_error(int e);
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kBlockK = 128;   // keys per dK/dV workgroup (32 per wave)
constexpr int kTileQ = 32;     // queries per dK/dV step
constexpr int kBlockQ = 128;   // queries per dQ workgroup (32 per wave)
#ifndef ATTN_CFG_BWD_DQ_TILE_K  // keys per dQ step; -D overrides it for a sweep
#define ATTN_CFG_BWD_DQ_TILE_K 64
#endif
constexpr int kTileK = ATTN_CFG_BWD_DQ_TILE_K;
static_assert(kTileK == 32 || kTileK == 64 || kTileK == 128, "dQ key tile");
#ifndef ATTN_CFG_BWD_LOOKAHEAD  // MFMA steps by which LDS operand reads run ahead
#define ATTN_CFG_BWD_LOOKAHEAD 2
#endif
constexpr int kBwdLookahead = ATTN_CFG_BWD_LOOKAHEAD;
static_assert(kBwdLookahead >= 1 && kBwdLookahead <= 3, "lookahead range");
constexpr float kLog2e = 1.4426950408889634f;
// Gradient stores with the non-temporal hint or plain. Each lane stores its own
// 8- or 16-byte pieces of a row, not whole cache lines, and streaming them past
// the caches measured 9% slower at the causal N=4096 d=128 workload: plain.
#ifndef ATTN_CFG_BWD_NONTEMPORAL
#define ATTN_CFG_BWD_NONTEMPORAL 0
#endif
// The dQ kernel's loads of O (each row read once, for D) with the
// non-temporal hint (1) or plain (0): the hint measured 0.7-3.4% slower.
#ifndef ATTN_CFG_BWD_O_NONTEMPORAL
#define ATTN_CFG_BWD_O_NONTEMPORAL 0
#endif

template <class T>
__device__ __forceinline__ void store_grad(T *dst, const T &val) {
  if (ATTN_CFG_BWD_NONTEMPORAL) __builtin_nontemporal_store(val, dst); else *dst = val;
}

struct BwdParams {
  const void *q, *k, *v, *o, *dout;
  const float *lse;  // [B][H][Nq] contiguous
  void *dq, *dk, *dv;
  f32x2 *ld;  // workspace: (L * log2 e, D) per query row, [B][H][Nq]
  // element strides of (batch, head, row) of each tensor; columns are unit-stride
  int64_t qs[3], ks[3], vs[3], os[3], dos[3], dqs[3], dks[3], dvs[3];
  int Nq, Nk;  // query rows and keys per head (equal when causal)
  int BH, H;
  int d;       // head dimension; columns d .. D-1 of the kernels read as zeros
  int o_f32;   // O is fp32 (else the input type)
  float qk;     // scale * log2(e)
  float scale;  // applied to dQ and dK
};

// Element offset of head bh = b * H + h in a tensor with strides st.
__device__ __forceinline__ int64_t head_off(const int64_t *st, int bh, int H) {
  const int b = bh / H;
  return (int64_t)b * st[0] + (int64_t)(bh - b * H) * st[1];
}

// ---------------------------------------------------------------------------
// LDS tiles: rows of D 16-bit elements, 16-byte chunks XOR-swizzled by row so
// that both reads below are free of bank conflicts:
//  - row reads (a lane takes 16 bytes of one row; 16 lanes read 16 rows);
//  - transposing reads (ds_read_b64_tr_b16: 16 lanes read 4 rows x 4
//    columns of 4 elements).
// The swizzle depends on the row modulo 16 only.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int row) {
  if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  const int r = (row >> 1) & 7;
  return ((r & 3) << 1) | (r >> 2);
}

// 16 bytes of row `row`, logical chunk `chunk` (elements 8*chunk .. +7).
template <int D>
__device__ __forceinline__ u32x4 row_frag(const uint16_t *tile, int row, int chunk) {
  return *reinterpret_cast<const u32x4 *>(tile + row * D + ((chunk ^ swz<D>(row)) << 3));
}

// Lane-constant offsets of the transposing reads: for column block cb and
// half u, the element offset (relative to row 16t) of the 4-element piece
// this lane supplies. In a 16-lane block (g, h) lane s = a + 4m supplies row
// 8u + 4g + m, columns 32cb + 16h + 4a .. +3.
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

// Operand of one 32x32x16 step contracting over 16 rows 16t .. 16t+15 of a
// row-major tile: lane l gets column 32cb + (l & 31) at rows
// 16t + 4g + 0..3 (k slots 8g + 0..3) and 16t + 8 + 4g + 0..3 (8g + 4..7),
// g = l >> 5 -- the row order of the 32x32 accumulator layout, so the other
// operand can come straight from an accumulator (acc_frag below).
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

template <int N, class Op, class Run>
__device__ __forceinline__ void pipelined(Op op, Run run) {
  mfma_pipelined<N, kBwdLookahead>(op, run);
}

struct FragPair {
  u32x4 a, b;
};

// fp32 pair -> packed bf16 / fp16, round to nearest even.
template <bool IS_BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (IS_BF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
  } else {
    f16x2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
  }
}

// Elements 8t .. 8t+7 of a 32x32 accumulator (rows 16t + 4g + 0..3 and
// 16t + 8 + 4g + 0..3 of the lane's column) as one 16-step operand.
template <bool IS_BF16>
__device__ __forceinline__ u32x4 acc_frag(const f32x16 &x, int t) {
  return u32x4{pack2<IS_BF16>(x[8 * t + 0], x[8 * t + 1]), pack2<IS_BF16>(x[8 * t + 2], x[8 * t + 3]),
               pack2<IS_BF16>(x[8 * t + 4], x[8 * t + 5]), pack2<IS_BF16>(x[8 * t + 6], x[8 * t + 7])};
}

template <bool IS_BF16>
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (IS_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Copies into LDS: buffer_load_dwordx4 ... lds moves 16 bytes per lane from
// the descriptor's range (reads past it return zeros) to LDS at M0 + 16*lane.
// Written as inline assembly so the compiler does not treat the copies in
// flight as writers of every LDS location; the kernels order them with an
// explicit vmcnt wait and a barrier.
// ---------------------------------------------------------------------------
constexpr int kBufferFlags = 0x00020000;  // word 3 of a raw buffer descriptor

__device__ __forceinline__ u32x4 make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xFFFFu,
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), (uint32_t)kBufferFlags};
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

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

constexpr uint32_t kOutOfRange = 0x80000000u;  // a source offset past any range

// Tile of R rows x D 16-bit elements of a matrix with row stride sn, copied by
// all THREADS threads: instruction c fills 16-byte slots c*THREADS + tid; slot s holds
// physical chunk s % CPR of tile row s / CPR, i.e. logical chunk
// (s % CPR) ^ swz(row). One instruction spans a whole number of swizzle
// periods (16 rows), so the lane's source offset is that of c = 0 plus c rows
// strides of RPI rows. A lane whose logical chunk starts at or past column d
// reads from an offset beyond the range, which returns zeros: the columns
// d .. D-1 of the tile are zero without any instruction in the loops.
template <int D, int R, int THREADS = kThreads>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = THREADS / CPR;  // rows per instruction
  static constexpr int INS = R / RPI;
  static_assert(INS * RPI == R && RPI % 16 == 0, "tile copy shape");
  uint32_t off0;  // source byte offset of instruction 0, or kOutOfRange
  uint32_t step;  // bytes between instructions: RPI rows
  __device__ void init(int tid, int64_t sn, int d) {
    const int row = tid / CPR, lc = (tid % CPR) ^ swz<D>(row);
    off0 = lc * 8 < d ? (uint32_t)(row * sn * 2 + lc * 16) : kOutOfRange;
    step = (uint32_t)(RPI * sn * 2);
  }
  // rows [r0, min(r0 + R, n)) of the matrix at `base` into the tile at `lds`.
  __device__ void issue(const uint16_t *base, int64_t sn, int r0, int n, int d, uint16_t *lds,
                        int wave) const {
    const int rows = min(n - r0, R);
    const uint32_t bytes = rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * sn + d) * 2) : 0u;
    const u32x4 rs = make_rsrc(base + (rows > 0 ? (int64_t)r0 * sn : 0), bytes);
    const uint32_t ldsb = __builtin_amdgcn_readfirstlane(lds_addr(lds) + wave * 64 * 16);
#pragma unroll
    for (int c = 0; c < INS; ++c)
      dma16(rs, ldsb + c * THREADS * 16, off0 == kOutOfRange ? kOutOfRange : off0 + c * step);
  }
};

// Halves of a packed fp16 pair as fp32 (exact).
__device__ __forceinline__ float f16_lo_to_f32(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi_to_f32(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// ---------------------------------------------------------------------------
// bwd_prep: LD[r] = (L_r * log2 e, D_r = sum_c dO[r,c] O[r,c]) for every
// query row r = bh * Nq + i (B*H*Nq rows). LPR lanes per row, 8 columns each
// (16 lanes for D = 128, 8 for D = 64); lanes whose columns start at or past d
// add nothing. IN is the element type of dO (attn_dtype: fp32, fp16 or bf16);
// O is that type or fp32.
// ---------------------------------------------------------------------------
template <int IN, bool NT = false>
__device__ __forceinline__ void load8(const void *base, int64_t e, float (&x)[8]) {
  if constexpr (IN == ATTN_F32) {
    const f32x4 *pa = reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + e);
    const f32x4 a = NT ? __builtin_nontemporal_load(pa) : *pa;
    const f32x4 b = NT ? __builtin_nontemporal_load(pa + 1) : pa[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = a[i], x[4 + i] = b[i];
  } else {
    const u32x4 *pw = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + e);
    const u32x4 w = NT ? __builtin_nontemporal_load(pw) : *pw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (IN == ATTN_BF16) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      } else {
        x[2 * i] = f16_lo_to_f32(w[i]);
        x[2 * i + 1] = f16_hi_to_f32(w[i]);
      }
    }
  }
}

// Eight packed 16-bit values (bf16 or fp16) as fp32 (exact).
template <bool IS_BF16>
__device__ __forceinline__ void unpack8(const u32x4 &w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (IS_BF16) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    } else {
      x[2 * i] = f16_lo_to_f32(w[i]);
      x[2 * i + 1] = f16_hi_to_f32(w[i]);
    }
  }
}

// sum_c dO_c O_c over the columns 16kc + 8g .. +7 (kc < NKC, below d) of one
// row: dO from the packed operands df, O (element type OT) read at ro. All
// loads are issued before the first product, so their latencies overlap.
template <int OT, int NKC, bool IS_BF16>
__device__ __forceinline__ float row_dot_o(const void *o, int64_t ro, const u32x4 *df, int g, int d) {
  float of[NKC][8];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    if (16 * kc + 8 * g < d) {
      load8<OT, ATTN_CFG_BWD_O_NONTEMPORAL>(o, ro + 16 * kc, of[kc]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) of[kc][c] = 0.f;
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    float dof[8];
    unpack8<IS_BF16>(df[kc], dof);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc += dof[c] * of[kc][c];
  }
  return acc;
}

template <int D, int IN, bool O_F32>
__global__ __launch_bounds__(256) void bwd_prep(BwdParams p, int64_t rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = gid / LPR;
  const int part = (int)(gid % LPR);
  float acc = 0.f;
  if (r < rows && part * 8 < p.d) {
    const int bh = (int)(r / p.Nq), i = (int)(r - (int64_t)bh * p.Nq);
    float dof[8], of[8];
    load8<IN>(p.dout, head_off(p.dos, bh, p.H) + (int64_t)i * p.dos[2] + part * 8, dof);
    load8<O_F32 ? (int)ATTN_F32 : IN>(p.o, head_off(p.os, bh, p.H) + (int64_t)i * p.os[2] + part * 8,
                                       of);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc += dof[c] * of[c];
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (r < rows && part == 0) p.ld[r] = f32x2{p.lse[r] * kLog2e, acc};
}

// ---------------------------------------------------------------------------
// bwd_dkdv
// ---------------------------------------------------------------------------
// WAVES waves of 32 keys each: 4 (two workgroups per CU), or 8 at D = 128 in
// a sweep build (one per CU).
template <int D, int WAVES>
struct DkdvShape {
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BLOCK_K = 32 * WAVES;        // keys per workgroup
  static constexpr int TILE = kTileQ * D;           // elements of a Q or dO tile
  static constexpr int STAGE = 2 * TILE + 512;      // Q, dO, LD (1 KB: one copy instruction)
  static constexpr int V_ELEMS = BLOCK_K * D;
  static constexpr int LDS_ELEMS = V_ELEMS + 2 * STAGE;
};

template <int D, bool IS_BF16, bool CAUSAL, bool GRAD_F32, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void bwd_dkdv(BwdParams p) {
  using S = DkdvShape<D, WAVES>;
  using QCopy = TileCopy<D, kTileQ, S::THREADS>;
  using VCopy = TileCopy<D, S::BLOCK_K, S::THREADS>;
  constexpr int NKC = D / 16, NCB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::LDS_ELEMS];

  // The wave index is read through a scalar register so that everything derived
  // from it (this wave's keys, the edge test below) is known to be wave-uniform
  // and branches on it are scalar branches, not per-lane masks.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int kbk = blockIdx.x / p.BH;  // small k0 first: causal blocks with most work start first
  const int bh = blockIdx.x - kbk * p.BH;
  const int Nq = p.Nq, Nk = p.Nk;
  const int k0 = kbk * S::BLOCK_K, kw0 = k0 + 32 * wave;
  const int d = p.d;
  const uint16_t *Qh = reinterpret_cast<const uint16_t *>(p.q) + head_off(p.qs, bh, p.H);
  const uint16_t *Kh = reinterpret_cast<const uint16_t *>(p.k) + head_off(p.ks, bh, p.H);
  const uint16_t *Vh = reinterpret_cast<const uint16_t *>(p.v) + head_off(p.vs, bh, p.H);
  const uint16_t *dOh = reinterpret_cast<const uint16_t *>(p.dout) + head_off(p.dos, bh, p.H);
  const f32x2 *LDh = p.ld + (size_t)bh * Nq;

  uint16_t *vlds = lds;
  auto stage = [&](int s) { return lds + S::V_ELEMS + s * S::STAGE; };

  QCopy qc, dc;
  qc.init(tid, p.qs[2], d);
  dc.init(tid, p.dos[2], d);
  const int q_begin = CAUSAL ? k0 : 0;
  const int n_qt = (Nq - q_begin + kTileQ - 1) / kTileQ;

  // Copies of query tile `it` into stage it & 1: Q and dO by every wave, LD by wave 0.
  auto issue = [&](int it) {
    const int q0 = q_begin + it * kTileQ;
    uint16_t *st = stage(it & 1);
    qc.issue(Qh, p.qs[2], q0, Nq, d, st, wave);
    dc.issue(dOh, p.dos[2], q0, Nq, d, st + S::TILE, wave);
    if (wave == 0) {
      const int rows = min(Nq - q0, kTileQ);
      const u32x4 rs = make_rsrc(LDh + q0, (uint32_t)rows * 8);
      dma16(rs, __builtin_amdgcn_readfirstlane(lds_addr(st + 2 * S::TILE)), lane * 16);
    }
  };

  // V block (this workgroup's keys) into LDS, and the first query tile.
  {
    VCopy vc;
    vc.init(tid, p.vs[2], d);
    vc.issue(Vh, p.vs[2], k0, Nk, d, vlds, wave);
  }
  issue(0);

  // K operand of S = Q K^T for this wave's keys: K[kw0 + l32][16kc + 8g ..].
  u32x4 kf[NKC];
  {
    const bool ok = kw0 + l32 < Nk;
    const uint16_t *kr = Kh + (int64_t)(ok ? kw0 + l32 : 0) * p.ks[2] + 8 * g;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
      kf[kc] = ok && 16 * kc + 8 * g < d ? *reinterpret_cast<const u32x4 *>(kr + 16 * kc)
                                         : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) settle(kf[kc]);
  }
  const TrAddr<D> ta = tr_addr<D>(lane);
  f32x16 dvt[NCB], dkt[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dvt[cb] = dkt[cb] = f32x16{};
  const int my_key = kw0 + l32;
  const float qk = p.qk;

#pragma unroll 1
  for (int it = 0; it < n_qt; ++it) {
    const int q0 = q_begin + it * kTileQ;
    // Tile it has landed (this wave's copies, then everyone's after the
    // barrier), and every wave is done with tile it - 1, whose stage the
    // copies of tile it + 1 then refill while tile it is computed: one
    // barrier per tile.
    wait_vmcnt<0>();
    lds_barrier();
    if (it + 1 < n_qt) issue(it + 1);
    const uint16_t *qt = stage(it & 1), *dot = qt + S::TILE;
    const f32x4 *ldt = reinterpret_cast<const f32x4 *>(qt + 2 * S::TILE);  // (L2, D) pairs
    // Whole tile above this wave's keys (causal): nothing to add.
    if (!CAUSAL || q0 + kTileQ - 1 >= kw0) {
      // S = Q K^T and dP = dO V^T: lane (key my_key) holds queries
      // q0 + 8j + 4g + r in element 4j + r of each.
      // Steps i < NKC: S += Q_kc K_kc^T (K from registers); the other NKC
      // steps: dP += dO_kc V_kc^T. LDS operands are read ahead (pipelined).
      f32x16 s = f32x16{}, dp = f32x16{};
      pipelined<2 * NKC>(
          [&](int i) {
            return i < NKC ? FragPair{row_frag<D>(qt, l32, 2 * i + g), kf[i]}
                           : FragPair{row_frag<D>(dot, l32, 2 * (i - NKC) + g),
                                      row_frag<D>(vlds, 32 * wave + l32, 2 * (i - NKC) + g)};
          },
          [&](int i, const FragPair &f) {
            if (i < NKC) s = mfma<IS_BF16>(f.a, f.b, s); else dp = mfma<IS_BF16>(f.a, f.b, dp);
          });
      // P = exp2(S * qk - L2) in place of S and dP - D in place of dP; masked
      // pairs (key after query, key or query past the end) get P = 0. Then
      // P and dS = P (dP - D) are packed as the operands of dV and dK.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 a = ldt[4 * j + 2 * g], b = ldt[4 * j + 2 * g + 1];  // rows 8j+4g .. +3
        const float l2[4] = {a[0], a[2], b[0], b[2]};
        const float dd[4] = {a[1], a[3], b[1], b[3]};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[4 * j + r] = __builtin_amdgcn_exp2f(s[4 * j + r] * qk - l2[r]);
          dp[4 * j + r] -= dd[r];
        }
      }
      // Only tiles on the diagonal or past an end hold masked pairs; the test
      // is wave-uniform, so interior tiles skip the masking entirely.
      if ((CAUSAL && q0 < kw0 + 32) || kw0 + 32 > Nk || q0 + kTileQ > Nq) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qrow = q0 + 8 * (e >> 2) + 4 * g + (e & 3);
          const bool keep = (!CAUSAL || my_key <= qrow) && my_key < Nk && qrow < Nq;
          s[e] = keep ? s[e] : 0.f;
        }
      }
      uint32_t pp[8], dsp[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pp[j] = pack2<IS_BF16>(s[2 * j], s[2 * j + 1]);
        dsp[j] = pack2<IS_BF16>(s[2 * j] * dp[2 * j], s[2 * j + 1] * dp[2 * j + 1]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS (operand t: elements 8t .. 8t+7)
      // Step i: operand t = i / (2 NCB), column block cb = (i / 2) % NCB, dV
      // for even i and dK for odd i; the transposing reads run ahead.
      pipelined<4 * NCB>(
          [&](int i) { return tr_frag<D>((i & 1) ? qt : dot, ta, i / (2 * NCB), (i >> 1) % NCB); },
          [&](int i, const u32x4 &a) {
            const int t = i / (2 * NCB), cb = (i >> 1) % NCB;
            if (i & 1) {
              const u32x4 df = {dsp[4 * t], dsp[4 * t + 1], dsp[4 * t + 2], dsp[4 * t + 3]};
              dkt[cb] = mfma<IS_BF16>(a, df, dkt[cb]);
            } else {
              const u32x4 pf = {pp[4 * t], pp[4 * t + 1], pp[4 * t + 2], pp[4 * t + 3]};
              dvt[cb] = mfma<IS_BF16>(a, pf, dvt[cb]);
            }
          });
    }
  }

  // dV^T / dK^T accumulators: lane holds key my_key, columns 32cb + 8j + 4g + 0..3.
  if (my_key < Nk) {
    const int64_t vrow = head_off(p.dvs, bh, p.H) + (int64_t)my_key * p.dvs[2];
    const int64_t krow = head_off(p.dks, bh, p.H) + (int64_t)my_key * p.dks[2];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 32 * cb + 8 * j + 4 * g;
        if (c >= d) continue;
        const f32x4 v4 = {dvt[cb][4 * j], dvt[cb][4 * j + 1], dvt[cb][4 * j + 2], dvt[cb][4 * j + 3]};
        const f32x4 k4 = {dkt[cb][4 * j] * p.scale, dkt[cb][4 * j + 1] * p.scale,
                          dkt[cb][4 * j + 2] * p.scale, dkt[cb][4 * j + 3] * p.scale};
        if constexpr (GRAD_F32) {
          store_grad(reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.dv) + vrow + c), v4);
          store_grad(reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.dk) + krow + c), k4);
        } else {
          store_grad(reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(p.dv) + vrow + c),
                     u32x2{pack2<IS_BF16>(v4[0], v4[1]), pack2<IS_BF16>(v4[2], v4[3])});
          store_grad(reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(p.dk) + krow + c),
                     u32x2{pack2<IS_BF16>(k4[0], k4[1]), pack2<IS_BF16>(k4[2], k4[3])});
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_dq
// ---------------------------------------------------------------------------
template <int D>
struct DqShape {
  static constexpr int TILE = kTileK * D;  // elements of a K or V tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int LDS_ELEMS = 2 * STAGE;
};

template <int D, bool IS_BF16, bool CAUSAL, bool GRAD_F32>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq(BwdParams p) {
  using S = DqShape<D>;
  using KCopy = TileCopy<D, kTileK>;
  constexpr int NKC = D / 16, NCB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::LDS_ELEMS];

  // Wave index through a scalar register: see bwd_dkdv.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int Nq = p.Nq, Nk = p.Nk;
  const int nqb = (Nq + kBlockQ - 1) / kBlockQ;
  const int t_ = blockIdx.x / p.BH;
  const int bh = blockIdx.x - t_ * p.BH;
  const int qb = CAUSAL ? nqb - 1 - t_ : t_;  // causal: longest first
  const int m0 = qb * kBlockQ, qw0 = m0 + 32 * wave;
  const int my_q = qw0 + l32;
  const int d = p.d;
  const uint16_t *Qh = reinterpret_cast<const uint16_t *>(p.q) + head_off(p.qs, bh, p.H);
  const uint16_t *Kh = reinterpret_cast<const uint16_t *>(p.k) + head_off(p.ks, bh, p.H);
  const uint16_t *Vh = reinterpret_cast<const uint16_t *>(p.v) + head_off(p.vs, bh, p.H);
  const uint16_t *dOh = reinterpret_cast<const uint16_t *>(p.dout) + head_off(p.dos, bh, p.H);

  KCopy kc_, vc_;
  kc_.init(tid, p.ks[2], d);
  vc_.init(tid, p.vs[2], d);
  const int kend = CAUSAL ? min(Nk, m0 + kBlockQ) : Nk;
  const int n_kt = (kend + kTileK - 1) / kTileK;
  auto stage = [&](int s) { return lds + s * S::STAGE; };
  auto issue = [&](int it) {
    uint16_t *st = stage(it & 1);
    kc_.issue(Kh, p.ks[2], it * kTileK, Nk, d, st, wave);
    vc_.issue(Vh, p.vs[2], it * kTileK, Nk, d, st + S::TILE, wave);
  };
  issue(0);

  // Q and dO operands of S^T = K Q^T and dP^T = V dO^T: row my_q, 16kc + 8g ..
  u32x4 qf[NKC], df[NKC];
  {
    const bool ok = my_q < Nq;
    const int64_t rq = (int64_t)(ok ? my_q : 0) * p.qs[2] + 8 * g;
    const int64_t rd = (int64_t)(ok ? my_q : 0) * p.dos[2] + 8 * g;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const bool in = ok && 16 * kc + 8 * g < d;
      qf[kc] = in ? *reinterpret_cast<const u32x4 *>(Qh + rq + 16 * kc) : u32x4{0, 0, 0, 0};
      df[kc] = in ? *reinterpret_cast<const u32x4 *>(dOh + rd + 16 * kc) : u32x4{0, 0, 0, 0};
    }
  }
  // This kernel runs first and does the preprocessing step for its rows:
  // D = sum_c dO_c O_c over the columns this lane holds in df (16kc + 8g ..
  // +7), the other half-wave's columns added by one swap, and L * log2 e.
  // Both go to LD for the dK/dV kernel that runs next.
  float dd = 0.f, l2 = 0.f;
  if (my_q < Nq) {
    const int64_t ro = head_off(p.os, bh, p.H) + (int64_t)my_q * p.os[2] + 8 * g;
    if (p.o_f32)
      dd = row_dot_o<ATTN_F32, NKC, IS_BF16>(p.o, ro, df, g, d);
    else
      dd = row_dot_o<IS_BF16 ? (int)ATTN_BF16 : (int)ATTN_F16, NKC, IS_BF16>(p.o, ro, df, g, d);
    l2 = p.lse[(size_t)bh * Nq + my_q] * kLog2e;
  }
  dd += __shfl_xor(dd, 32);
  if (g == 0 && my_q < Nq) p.ld[(size_t)bh * Nq + my_q] = f32x2{l2, dd};
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    settle(qf[kc]);
    settle(df[kc]);
  }
  const TrAddr<D> ta = tr_addr<D>(lane);
  f32x16 dqt[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dqt[cb] = f32x16{};
  const float qk = p.qk;

#pragma unroll 1
  for (int it = 0; it < n_kt; ++it) {
    // As in bwd_dkdv: wait for tile it, one barrier, then refill the stage of
    // tile it - 1 with tile it + 1 while tile it is computed.
    wait_vmcnt<0>();
    lds_barrier();
    if (it + 1 < n_kt) issue(it + 1);
    const uint16_t *kt = stage(it & 1), *vt = kt + S::TILE;
#pragma unroll
    for (int kb = 0; kb < kTileK / 32; ++kb) {
      const int key0 = it * kTileK + 32 * kb;
      if (CAUSAL && key0 > qw0 + 31) continue;  // every key after every query of this wave
      // S^T = K Q^T: lane (query my_q) holds keys key0 + 8j + 4g + r in s[4j + r].
      // Steps i < NKC: S^T += K_kc Q_kc^T; the other NKC: dP^T += V_kc dO_kc^T
      // (Q and dO from registers). The LDS operand is read ahead.
      f32x16 s = f32x16{}, dp = f32x16{};
      pipelined<2 * NKC>(
          [&](int i) { return row_frag<D>(i < NKC ? kt : vt, 32 * kb + l32, 2 * (i % NKC) + g); },
          [&](int i, const u32x4 &a) {
            if (i < NKC) s = mfma<IS_BF16>(a, qf[i], s); else dp = mfma<IS_BF16>(a, df[i - NKC], dp);
          });
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = __builtin_amdgcn_exp2f(s[e] * qk - l2);  // P
      // Masked pairs only on the diagonal or past the last key (wave-uniform test).
      if ((CAUSAL && key0 + 31 > qw0) || key0 + 32 > Nk) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + 8 * (e >> 2) + 4 * g + (e & 3);
          const bool keep = (!CAUSAL || key <= my_q) && key < Nk;
          s[e] = keep ? s[e] : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) dp[e] = s[e] * (dp[e] - dd);  // dS
      // dQ^T += K^T dS^T
      {
        const uint16_t *kk = kt + 32 * kb * D;
        const u32x4 sf[2] = {acc_frag<IS_BF16>(dp, 0), acc_frag<IS_BF16>(dp, 1)};
        pipelined<2 * NCB>(  // step i: t = i / NCB, cb = i % NCB
            [&](int i) { return tr_frag<D>(kk, ta, i / NCB, i % NCB); },
            [&](int i, const u32x4 &a) { dqt[i % NCB] = mfma<IS_BF16>(a, sf[i / NCB], dqt[i % NCB]); });
      }
    }
  }

  // dQ^T accumulators: lane holds query my_q, columns 32cb + 8j + 4g + 0..3.
  if (my_q < Nq) {
    const int64_t row = head_off(p.dqs, bh, p.H) + (int64_t)my_q * p.dqs[2];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 32 * cb + 8 * j + 4 * g;
        if (c >= d) continue;
        const f32x4 q4 = {dqt[cb][4 * j] * p.scale, dqt[cb][4 * j + 1] * p.scale,
                          dqt[cb][4 * j + 2] * p.scale, dqt[cb][4 * j + 3] * p.scale};
        if constexpr (GRAD_F32)
          store_grad(reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.dq) + row + c), q4);
        else
          store_grad(reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(p.dq) + row + c),
                     u32x2{pack2<IS_BF16>(q4[0], q4[1]), pack2<IS_BF16>(q4[2], q4[3])});
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs (the page's check of the backward in fp32): the same split on
// v_mfma_f32_32x32x2_f32, everything in fp32. Tiles of 32 rows go through LDS
// with plain strided loads (rows of D + 2 floats: the row-per-lane operand
// reads hit 32 different banks); columns past d read as zeros.
//
// Contractions whose operand sits in a score tile held row-per-lane take
// that tile straight from the registers: in a 32x32 accumulator, lane
// (l32, g) holds element r of its column at row 8(r/4) + 4g + r%4, so step s
// (of 16) of the contraction pairs k slot g with row 8(s/4) + 4g + s%4, and
// the other operand is read from LDS at that row.
// ---------------------------------------------------------------------------
template <int D>
struct F32Tile {
  static constexpr int STR = D + 2;   // floats per LDS row
  static constexpr int ELEMS = 32 * STR;
};

// Rows r0 .. r0+31 (those < n) of a strided fp32 matrix into an LDS tile;
// other rows and columns >= d are zero.
template <int D>
__device__ __forceinline__ void load_tile_f32(float *t, const float *base, int64_t sn, int r0, int n,
                                              int d, int tid) {
  for (int e = tid; e < 32 * D / 4; e += kThreads) {
    const int row = e / (D / 4), c = (e % (D / 4)) * 4;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (r0 + row < n && c < d) x = *reinterpret_cast<const f32x4 *>(base + (int64_t)(r0 + row) * sn + c);
    float *dst = t + row * F32Tile<D>::STR + c;
    dst[0] = x[0], dst[1] = x[1], dst[2] = x[2], dst[3] = x[3];
  }
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// dK, dV: one workgroup per (head, 128 keys), 4 waves x 32 keys; per 32-query
// tile S = Q K^T and dP = dO V^T (lane: one key, 16 queries), P, dS, then
// dV^T += dO^T P and dK^T += Q^T dS with P and dS from the registers.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_f32(BwdParams p) {
  constexpr int NCB = D / 32, STR = F32Tile<D>::STR;
  __shared__ float qt[F32Tile<D>::ELEMS], dot[F32Tile<D>::ELEMS];
  __shared__ f32x2 ldt[32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int kbk = blockIdx.x / p.BH, bh = blockIdx.x - kbk * p.BH;
  const int Nq = p.Nq, Nk = p.Nk, d = p.d;
  const int k0 = kbk * kBlockK, kw0 = k0 + 32 * wave, my_key = kw0 + l32;
  const float *Qh = static_cast<const float *>(p.q) + head_off(p.qs, bh, p.H);
  const float *Kh = static_cast<const float *>(p.k) + head_off(p.ks, bh, p.H);
  const float *Vh = static_cast<const float *>(p.v) + head_off(p.vs, bh, p.H);
  const float *dOh = static_cast<const float *>(p.dout) + head_off(p.dos, bh, p.H);
  const f32x2 *LDh = p.ld + (size_t)bh * Nq;
  // K and V operands: row my_key, columns 2kk + g
  float kf[D / 2], vf[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) {
    const int c = 2 * kk + g;
    const bool ok = my_key < Nk && c < d;
    kf[kk] = ok ? Kh[(int64_t)my_key * p.ks[2] + c] : 0.f;
    vf[kk] = ok ? Vh[(int64_t)my_key * p.vs[2] + c] : 0.f;
  }
  f32x16 dvt[NCB], dkt[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dvt[cb] = dkt[cb] = f32x16{};
  const float qk = p.qk;
  const int q_begin = CAUSAL ? k0 : 0;
#pragma unroll 1
  for (int q0 = q_begin; q0 < Nq; q0 += 32) {
    __syncthreads();  // the previous tile is consumed
    load_tile_f32<D>(qt, Qh, p.qs[2], q0, Nq, d, tid);
    load_tile_f32<D>(dot, dOh, p.dos[2], q0, Nq, d, tid);
    if (tid < 32) ldt[tid] = q0 + tid < Nq ? LDh[q0 + tid] : f32x2{0.f, 0.f};
    __syncthreads();
    if (CAUSAL && q0 + 31 < kw0) continue;  // every query before every key of this wave
    f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
      sc = mfma_f32(qt[l32 * STR + 2 * kk + g], kf[kk], sc);
      dp = mfma_f32(dot[l32 * STR + 2 * kk + g], vf[kk], dp);
    }
    // element r: query q0 + 8(r/4) + 4g + r%4, key my_key
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = 8 * (r >> 2) + 4 * g + (r & 3), qrow = q0 + qi;
      const f32x2 ld = ldt[qi];
      const bool keep = qrow < Nq && my_key < Nk && (!CAUSAL || my_key <= qrow);
      const float pw = keep ? __builtin_amdgcn_exp2f(sc[r] * qk - ld[0]) : 0.f;
      sc[r] = pw;                    // P
      dp[r] = pw * (dp[r] - ld[1]);  // dS
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const int qi = 8 * (st >> 2) + 4 * g + (st & 3);
        dvt[cb] = mfma_f32(dot[qi * STR + 32 * cb + l32], sc[st], dvt[cb]);
        dkt[cb] = mfma_f32(qt[qi * STR + 32 * cb + l32], dp[st], dkt[cb]);
      }
  }
  // dV^T / dK^T: lane holds key my_key, columns 32cb + 8j + 4g + 0..3
  if (my_key < Nk) {
    float *dvr = static_cast<float *>(p.dv) + head_off(p.dvs, bh, p.H) + (int64_t)my_key * p.dvs[2];
    float *dkr = static_cast<float *>(p.dk) + head_off(p.dks, bh, p.H) + (int64_t)my_key * p.dks[2];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 32 * cb + 8 * j + 4 * g;
        if (c >= d) continue;
        *reinterpret_cast<f32x4 *>(dvr + c) =
            f32x4{dvt[cb][4 * j], dvt[cb][4 * j + 1], dvt[cb][4 * j + 2], dvt[cb][4 * j + 3]};
        *reinterpret_cast<f32x4 *>(dkr + c) =
            f32x4{dkt[cb][4 * j] * p.scale, dkt[cb][4 * j + 1] * p.scale,
                  dkt[cb][4 * j + 2] * p.scale, dkt[cb][4 * j + 3] * p.scale};
      }
  }
}

// dQ: one workgroup per (head, 128 queries), 4 waves x 32 queries; per
// 32-key tile S^T = K Q^T and dP^T = V dO^T (lane: one query, 16 keys), P,
// dS, then dQ^T += K^T dS^T with dS from the registers.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_f32(BwdParams p) {
  constexpr int NCB = D / 32, STR = F32Tile<D>::STR;
  __shared__ float kt[F32Tile<D>::ELEMS], vt[F32Tile<D>::ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int Nq = p.Nq, Nk = p.Nk, d = p.d;
  const int nqb = (Nq + kBlockQ - 1) / kBlockQ;
  const int t_ = blockIdx.x / p.BH, bh = blockIdx.x - t_ * p.BH;
  const int qb = CAUSAL ? nqb - 1 - t_ : t_;  // causal: longest first
  const int m0 = qb * kBlockQ, qw0 = m0 + 32 * wave, my_q = qw0 + l32;
  const float *Qh = static_cast<const float *>(p.q) + head_off(p.qs, bh, p.H);
  const float *Kh = static_cast<const float *>(p.k) + head_off(p.ks, bh, p.H);
  const float *Vh = static_cast<const float *>(p.v) + head_off(p.vs, bh, p.H);
  const float *dOh = static_cast<const float *>(p.dout) + head_off(p.dos, bh, p.H);
  float qf[D / 2], df[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) {
    const int c = 2 * kk + g;
    const bool ok = my_q < Nq && c < d;
    qf[kk] = ok ? Qh[(int64_t)my_q * p.qs[2] + c] : 0.f;
    df[kk] = ok ? dOh[(int64_t)my_q * p.dos[2] + c] : 0.f;
  }
  const f32x2 ldv = my_q < Nq ? p.ld[(size_t)bh * Nq + my_q] : f32x2{0.f, 0.f};
  f32x16 dqt[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dqt[cb] = f32x16{};
  const float qk = p.qk;
  const int kend = CAUSAL ? min(Nk, m0 + kBlockQ) : Nk;
#pragma unroll 1
  for (int key0 = 0; key0 < kend; key0 += 32) {
    __syncthreads();
    load_tile_f32<D>(kt, Kh, p.ks[2], key0, Nk, d, tid);
    load_tile_f32<D>(vt, Vh, p.vs[2], key0, Nk, d, tid);
    __syncthreads();
    if (CAUSAL && key0 > qw0 + 31) continue;  // every key after every query of this wave
    f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
      sc = mfma_f32(kt[l32 * STR + 2 * kk + g], qf[kk], sc);
      dp = mfma_f32(vt[l32 * STR + 2 * kk + g], df[kk], dp);
    }
    // element r: key key0 + 8(r/4) + 4g + r%4, query my_q
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * g + (r & 3);
      const bool keep = key < Nk && my_q < Nq && (!CAUSAL || key <= my_q);
      const float pw = keep ? __builtin_amdgcn_exp2f(sc[r] * qk - ldv[0]) : 0.f;
      dp[r] = pw * (dp[r] - ldv[1]);  // dS
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const int ki = 8 * (st >> 2) + 4 * g + (st & 3);
        dqt[cb] = mfma_f32(kt[ki * STR + 32 * cb + l32], dp[st], dqt[cb]);
      }
  }
  if (my_q < Nq) {
    float *dqr = static_cast<float *>(p.dq) + head_off(p.dqs, bh, p.H) + (int64_t)my_q * p.dqs[2];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 32 * cb + 8 * j + 4 * g;
        if (c >= d) continue;
        *reinterpret_cast<f32x4 *>(dqr + c) =
            f32x4{dqt[cb][4 * j] * p.scale, dqt[cb][4 * j + 1] * p.scale,
                  dqt[cb][4 * j + 2] * p.scale, dqt[cb][4 * j + 3] * p.scale};
      }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
typedef void (*KernelFn)(BwdParams);
typedef void (*PrepFn)(BwdParams, int64_t);

// Waves per dK/dV workgroup for 16-bit inputs. 8 (at D = 128 only: one
// workgroup per CU, each Q and dO tile in LDS serving 256 keys) measured
// 0.4-5.5% slower than 4 at every d = 128 workload timed, so 4 ships and the
// 8-wave kernels are built only for a sweep (-DATTN_CFG_BWD_DKDV_WAVES=8).
#ifndef ATTN_CFG_BWD_DKDV_WAVES
#define ATTN_CFG_BWD_DKDV_WAVES 4
#endif
static_assert(ATTN_CFG_BWD_DKDV_WAVES == 4 || ATTN_CFG_BWD_DKDV_WAVES == 8, "dK/dV waves");

template <int D, bool IS_BF16, bool CAUSAL, bool GRAD_F32>
void pick3(int waves, KernelFn &dkdv, KernelFn &dq) {
  dkdv = bwd_dkdv<D, IS_BF16, CAUSAL, GRAD_F32, 4>;
  if constexpr (D == 128 && ATTN_CFG_BWD_DKDV_WAVES == 8)
    if (waves == 8) dkdv = bwd_dkdv<D, IS_BF16, CAUSAL, GRAD_F32, 8>;
  dq = bwd_dq<D, IS_BF16, CAUSAL, GRAD_F32>;
}

template <int D, bool IS_BF16>
void pick2(bool causal, bool grad_f32, int waves, KernelFn &dkdv, KernelFn &dq) {
  if (causal) {
    if (grad_f32) pick3<D, IS_BF16, true, true>(waves, dkdv, dq);
    else pick3<D, IS_BF16, true, false>(waves, dkdv, dq);
  } else {
    if (grad_f32) pick3<D, IS_BF16, false, true>(waves, dkdv, dq);
    else pick3<D, IS_BF16, false, false>(waves, dkdv, dq);
  }
}

// The 8-wave build takes D = 128 problems whose V block of 256 rows spans
// less than 2^31 bytes.
int dkdv_waves(int64_t D, int64_t v_row_bytes) {
  return ATTN_CFG_BWD_DKDV_WAVES == 8 && D == 128 && v_row_bytes * 256 < (int64_t(1) << 31) ? 8 : 4;
}

template <int D>
void pick_f32(bool causal, KernelFn &dkdv, KernelFn &dq) {
  dkdv = causal ? bwd_dkdv_f32<D, true> : bwd_dkdv_f32<D, false>;
  dq = causal ? bwd_dq_f32<D, true> : bwd_dq_f32<D, false>;
}


size_t ws_bytes(int64_t B, int64_t H, int64_t N) {
  return (((size_t)(B * H) * (size_t)N * 8) + 255) & ~(size_t)255;
}

int elem_bytes(attn_dtype t) { return t == ATTN_F32 ? 4 : 2; }

// Element strides of the (batch, head, row) dimensions of every tensor.
struct BwdViews {
  int64_t qs[3], ks[3], vs[3], os[3], dos[3], dqs[3], dks[3], dvs[3];
};

// The given strides, or those of a contiguous [B][H][n][d] tensor.
void fill_strides(int64_t out[3], const int64_t *in, int64_t H, int64_t n, int64_t d) {
  if (in) {
    out[0] = in[0], out[1] = in[1], out[2] = in[2];
  } else {
    out[2] = d, out[1] = n * d, out[0] = H * n * d;
  }
}

BwdViews contiguous_views(int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
  BwdViews w;
  fill_strides(w.qs, nullptr, H, Nq, d);
  fill_strides(w.ks, nullptr, H, Nk, d);
  fill_strides(w.vs, nullptr, H, Nk, d);
  fill_strides(w.os, nullptr, H, Nq, d);
  fill_strides(w.dos, nullptr, H, Nq, d);
  fill_strides(w.dqs, nullptr, H, Nq, d);
  fill_strides(w.dks, nullptr, H, Nk, d);
  fill_strides(w.dvs, nullptr, H, Nk, d);
  return w;
}

// A strided view is usable when every offset is non-negative and below 2^47
// elements, rows do not overlap (row stride >= d), every row starts 16-byte
// aligned, and a tile of 128 rows spans less than 2^31 bytes (the range of a
// buffer descriptor).
bool view_ok(const void *ptr, const int64_t s[3], int64_t B, int64_t H, int64_t n, int64_t d,
             int eb) {
  if (s[0] < 0 || s[1] < 0 || s[2] < d) return false;
  const int64_t lim = int64_t(1) << 47;
  if (s[0] > lim / B || s[1] > lim / H || s[2] > lim / n) return false;
  if ((reinterpret_cast<uintptr_t>(ptr) & 15) != 0) return false;
  for (int i = 0; i < 3; ++i)
    if ((s[i] * eb) % 16 != 0) return false;
  return s[2] * eb * 128 < (int64_t(1) << 31);
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

// Argument checks shared by the backward's entry points; no HIP call.
attn_status bwd_check(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, const void *dout, void *dq, void *dk, void *dv,
                      int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                      float scale, attn_dtype in_dtype, attn_dtype o_dtype,
                      attn_dtype grad_dtype) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_ERR_SHAPE;
  if (Nq > (int64_t(1) << 24) || Nk > (int64_t(1) << 24) || B * H > (int64_t(1) << 24))
    return ATTN_ERR_SHAPE;
  if (causal && Nq != Nk) return ATTN_ERR_SHAPE;
  if (d < 8 || d > 128 || d % 8 != 0) return ATTN_ERR_UNSUPPORTED;
  if (in_dtype == ATTN_F32) {
    if (o_dtype != ATTN_F32 || grad_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  } else {
    if (in_dtype != ATTN_BF16 && in_dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
    if (o_dtype != in_dtype && o_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
    if (grad_dtype != in_dtype && grad_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  }
  if (!(scale >= 0.f) || !isfinite(scale)) return ATTN_ERR_SCALE;
  return ATTN_OK;
}

// Checks of the eight views (strided entry point).
attn_status views_check(const void *q, const void *k, const void *v, const void *o,
                        const void *dout, const void *dq, const void *dk, const void *dv,
                        const BwdViews &w, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                        int64_t d, attn_dtype in_dtype, attn_dtype o_dtype,
                        attn_dtype grad_dtype) {
  const int ei = elem_bytes(in_dtype), eo = elem_bytes(o_dtype), eg = elem_bytes(grad_dtype);
  if (!view_ok(q, w.qs, B, H, Nq, d, ei) || !view_ok(k, w.ks, B, H, Nk, d, ei) ||
      !view_ok(v, w.vs, B, H, Nk, d, ei) || !view_ok(o, w.os, B, H, Nq, d, eo) ||
      !view_ok(dout, w.dos, B, H, Nq, d, ei) || !view_ok(dq, w.dqs, B, H, Nq, d, eg) ||
      !view_ok(dk, w.dks, B, H, Nk, d, eg) || !view_ok(dv, w.dvs, B, H, Nk, d, eg) ||
      !out_view_disjoint(w.dqs, B, H, Nq, d) || !out_view_disjoint(w.dks, B, H, Nk, d) ||
      !out_view_disjoint(w.dvs, B, H, Nk, d))
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// The launches, with LD rows (8 bytes per query row) at `ld`. Checks the
// launch sizes before any HIP call.
attn_status bwd_run(const void *q, const void *k, const void *v, const void *o,
                    const float *lse, const void *dout, void *dq, void *dk, void *dv,
                    const BwdViews &w, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                    int causal, float scale, attn_dtype in_dtype, attn_dtype o_dtype,
                    attn_dtype grad_dtype, void *ld, void *stream) {
  const int64_t D = d <= 64 ? 64 : 128;  // the kernels' head dim; columns past d are zeros
  const int waves = in_dtype == ATTN_F32 ? 4 : dkdv_waves(D, w.vs[2] * elem_bytes(in_dtype));
  const int64_t block_k = 32 * waves;  // keys per dK/dV workgroup
  const int64_t nkb = (Nk + block_k - 1) / block_k, nqb = (Nq + kBlockQ - 1) / kBlockQ;
  const int64_t rows = B * H * Nq;
  const int64_t lpr = D / 8;
  const int64_t prep_blocks = (rows * lpr + 255) / 256;
  if (nkb * B * H > INT32_MAX || nqb * B * H > INT32_MAX || prep_blocks > INT32_MAX)
    return ATTN_ERR_SHAPE;

  BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.ld = reinterpret_cast<f32x2 *>(ld);
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = w.qs[i], p.ks[i] = w.ks[i], p.vs[i] = w.vs[i], p.os[i] = w.os[i];
    p.dos[i] = w.dos[i], p.dqs[i] = w.dqs[i], p.dks[i] = w.dks[i], p.dvs[i] = w.dvs[i];
  }
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.BH = (int)(B * H);
  p.H = (int)H;
  p.d = (int)d;
  p.o_f32 = o_dtype == ATTN_F32;
  p.qk = (float)((double)scale * 1.4426950408889634);
  p.scale = scale;

  const bool grad_f32 = grad_dtype == ATTN_F32;
  KernelFn fdkdv, fdq;
  if (in_dtype == ATTN_F32) {
    if (D == 64) pick_f32<64>(causal != 0, fdkdv, fdq); else pick_f32<128>(causal != 0, fdkdv, fdq);
  } else if (D == 64) {
    if (in_dtype == ATTN_BF16) pick2<64, true>(causal != 0, grad_f32, waves, fdkdv, fdq);
    else pick2<64, false>(causal != 0, grad_f32, waves, fdkdv, fdq);
  } else {
    if (in_dtype == ATTN_BF16) pick2<128, true>(causal != 0, grad_f32, waves, fdkdv, fdq);
    else pick2<128, false>(causal != 0, grad_f32, waves, fdkdv, fdq);
  }
  hipStream_t st = (hipStream_t)stream;
  void *args[] = {&p};
  hipError_t err = hipSuccess;
  if (in_dtype == ATTN_F32) {
    // prep, then dK/dV and dQ
    int64_t rows_arg = rows;
    void *pargs[] = {&p, &rows_arg};
    const PrepFn fprep = D == 64 ? bwd_prep<64, ATTN_F32, true> : bwd_prep<128, ATTN_F32, true>;
    err = hipLaunchKernel(reinterpret_cast<const void *>(fprep), dim3((unsigned)prep_blocks),
                          dim3(256), pargs, 0, st);
    if (err == hipSuccess)
      err = hipLaunchKernel(reinterpret_cast<const void *>(fdkdv), dim3((unsigned)(nkb * B * H)),
                            dim3(kThreads), args, 0, st);
    if (err == hipSuccess)
      err = hipLaunchKernel(reinterpret_cast<const void *>(fdq), dim3((unsigned)(nqb * B * H)),
                            dim3(kThreads), args, 0, st);
  } else {
    // dQ (which writes LD for its rows), then dK/dV
    err = hipLaunchKernel(reinterpret_cast<const void *>(fdq), dim3((unsigned)(nqb * B * H)),
                          dim3(kThreads), args, 0, st);
    if (err == hipSuccess)
      err = hipLaunchKernel(reinterpret_cast<const void *>(fdkdv), dim3((unsigned)(nkb * B * H)),
                            dim3((unsigned)(64 * waves)), args, 0, st);
  }
  if (err != hipSuccess) {
    attn_internal::set_last_hip_error((int)err);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

// The allocation-free backward (attn_bwd_noalloc) keeps its LD rows in this
// array instead of a caller's workspace: one copy per GPU, held until the
// process ends. Host code never uses the name itself (on the host it is a
// stand-in, not a device address): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = size_t(16) << 20;  // 2^21 query rows of 8 bytes
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on first use).
attn_status scratch_address(void **out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess && (dev < 0 || dev >= kMaxDevices)) err = hipErrorInvalidDevice;
  if (err != hipSuccess) {
    attn_internal::set_last_hip_error((int)err);
    return ATTN_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !ptr) {
      attn_internal::set_last_hip_error((int)(err != hipSuccess ? err : hipErrorInvalidSymbol));
      return ATTN_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  if (B < 1 || H < 1 || N < 1 || N > (int64_t(1) << 24) || B * H > (int64_t(1) << 24)) return 0;
  if (d < 8 || d > 128 || d % 8 != 0) return 0;
  return ws_bytes(B, H, N);
}

attn_status attn_bwd_qk(const void *q, const void *k, const void *v, const void *o,
                        const float *lse, const void *dout, void *dq, void *dk, void *dv,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                        float scale, attn_dtype in_dtype, attn_dtype o_dtype,
                        attn_dtype grad_dtype, void *workspace, size_t workspace_bytes,
                        void *stream) {
  // Validation first: no HIP call happens before every argument is checked.
  attn_status st = bwd_check(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, causal, scale,
                             in_dtype, o_dtype, grad_dtype);
  if (st != ATTN_OK) return st;
  const size_t need = ws_bytes(B, H, Nq);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
    return ATTN_ERR_WORKSPACE;
  return bwd_run(q, k, v, o, lse, dout, dq, dk, dv, contiguous_views(H, Nq, Nk, d), B, H, Nq, Nk,
                 d, causal, scale, in_dtype, o_dtype, grad_dtype, workspace, stream);
}

attn_status attn_bwd_strided(const void *q, const int64_t *q_strides, const void *k,
                             const int64_t *k_strides, const void *v, const int64_t *v_strides,
                             const void *o, const int64_t *o_strides, const float *lse,
                             const void *dout, const int64_t *dout_strides, void *dq,
                             const int64_t *dq_strides, void *dk, const int64_t *dk_strides,
                             void *dv, const int64_t *dv_strides, int64_t B, int64_t H,
                             int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                             attn_dtype in_dtype, attn_dtype o_dtype, attn_dtype grad_dtype,
                             void *workspace, size_t workspace_bytes, void *stream) {
  attn_status st = bwd_check(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, causal, scale,
                             in_dtype, o_dtype, grad_dtype);
  if (st != ATTN_OK) return st;
  BwdViews w;
  fill_strides(w.qs, q_strides, H, Nq, d);
  fill_strides(w.ks, k_strides, H, Nk, d);
  fill_strides(w.vs, v_strides, H, Nk, d);
  fill_strides(w.os, o_strides, H, Nq, d);
  fill_strides(w.dos, dout_strides, H, Nq, d);
  fill_strides(w.dqs, dq_strides, H, Nq, d);
  fill_strides(w.dks, dk_strides, H, Nk, d);
  fill_strides(w.dvs, dv_strides, H, Nk, d);
  st = views_check(q, k, v, o, dout, dq, dk, dv, w, B, H, Nq, Nk, d, in_dtype, o_dtype, grad_dtype);
  if (st != ATTN_OK) return st;
  const size_t need = ws_bytes(B, H, Nq);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
    return ATTN_ERR_WORKSPACE;
  return bwd_run(q, k, v, o, lse, dout, dq, dk, dv, w, B, H, Nq, Nk, d, causal, scale, in_dtype,
                 o_dtype, grad_dtype, workspace, stream);
}

attn_status attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                             const float *lse, const void *dout, void *dq, void *dk, void *dv,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                             float scale, attn_dtype in_dtype, attn_dtype o_dtype,
                             attn_dtype grad_dtype, void *stream) {
  attn_status st = bwd_check(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, causal, scale,
                             in_dtype, o_dtype, grad_dtype);
  if (st != ATTN_OK) return st;
  if (ws_bytes(B, H, Nq) > kScratchBytes) return ATTN_ERR_CAPACITY;
  void *ld = nullptr;
  st = scratch_address(&ld);
  if (st != ATTN_OK) return st;
  return bwd_run(q, k, v, o, lse, dout, dq, dk, dv, contiguous_views(H, Nq, Nk, d), B, H, Nq, Nk,
                 d, causal, scale, in_dtype, o_dtype, grad_dtype, ld, stream);
}

attn_status attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                     const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H,
                     int64_t N, int64_t d, int causal, float scale, attn_dtype in_dtype,
                     attn_dtype o_dtype, attn_dtype grad_dtype, void *workspace,
                     size_t workspace_bytes, void *stream) {
  return attn_bwd_qk(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, N, d, causal, scale, in_dtype,
                     o_dtype, grad_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"
