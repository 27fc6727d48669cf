// Attention forward for gfx950 (MI355X, CDNA4): HIP kernels and the C ABI
// declared in include/attn.h.
//
// The method is the FlashAttention forward of "4.4 Writing GPU Kernels with
// Triton" (section "Kernel 4: A Simplified FlashAttention"): one workgroup
// owns a block of query rows, keeps it resident, streams the keys/values of
// its (batch, head) tile by tile and maintains per row the running maximum
// m, the running sum l and the rescaled fp32 output accumulator (section
// "The Online Softmax Recurrence"). The score matrix never leaves the chip.
// Scores are kept in base-2 units (scale * log2 e folded into one factor) so
// every exponential is a single v_exp_f32, and the stored LSE is converted
// back to the natural log ("Kernel 4", notes on exp2 and the saved L).
//
// gfx950 mapping (our design, not the page's):
//  * a workgroup is 4 wave64s and 128 query rows; each wave owns 32 rows.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16}: with the 32x32 output
//    layout each lane then holds the scores of ONE query row (lane & 31) for
//    16 keys per 32-key block, so the row maximum is an in-lane max plus one
//    exchange with lane ^ 32, and the row sum needs no exchange until the
//    end.
//  * O^T += V^T P^T on v_mfma_f32_32x32x16_f16: the B operand P^T comes
//    straight from the S^T accumulators of the same lane (converted to
//    fp16), and the O^T accumulator has the same row-per-lane layout, so
//    rescaling by alpha is a per-lane scalar multiply.
//  * K tiles are staged in LDS as they are in memory (row-major, 16-byte
//    padded rows); V tiles are written to LDS transposed (V^T, key-permuted
//    so each lane's eight keys are contiguous) and, for bf16 inputs,
//    converted to fp16 on the way. Both are double-buffered: the global
//    loads of tile j+1 are in flight while tile j is computed.
//  * fp32 inputs use a separate kernel on v_mfma_f32_32x32x2_f32.
#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 kernel shape (the bf16/fp16 kernel defines its own below).
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = 128;  // query rows per workgroup (32 per wave)

struct FwdParams {
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;
  int N;         // sequence length
  int nq;        // query tiles per (batch, head)
  int BH;        // batch * heads
  float qk;      // scale * log2(e), >= FLT_MIN
};

// Work item of this workgroup: (bh, query tile). Workgroups are dispatched
// in id order and handed to the 8 XCDs round-robin, so id w runs on XCD
// w % 8. Ids are enumerated tile-major, head-minor: causal tiles go longest
// first across all heads (greedy longest-first keeps the tail short), and
// when B*H is a multiple of 8 every tile of head bh runs on XCD bh % 8,
// where its K/V stay in that XCD's L2.
template <bool CAUSAL>
__device__ __forceinline__ void work_item(const FwdParams &p, int &bh, int &qt) {
  const int w = blockIdx.x;
  const int t = w / p.BH;
  bh = w - t * p.BH;
  qt = CAUSAL ? p.nq - 1 - t : t;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float shfl_xor32(float x) { return __shfl_xor(x, 32); }

// --------------------------------------------------------------------------
// bf16 / fp16 kernel
// --------------------------------------------------------------------------
constexpr int kThreads16 = kThreads;  // 4 waves, 128 query rows per workgroup
constexpr int kBlockM16 = kBlockM;
// Tile shapes: D=128 uses BN=64 keys per tile, D=64 uses BN=128, so that one
// thread moves exactly one 4-key x 8-column unit of V per tile.
template <int D>
struct Shape16 {
  static constexpr int BN = (D == 128) ? 64 : 128;
  static constexpr int KSTR = D + 8;   // K row stride in LDS (elements), 16 B pad
  static constexpr int VSTR = BN + 8;  // V^T row stride in LDS (elements), 16 B pad
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int K_CHUNKS = BN * D / 8 / kThreads;  // 16-byte K chunks per thread
  static constexpr int KG = BN / 4;                        // 4-key groups per tile
  static constexpr int NKB = BN / 32;                      // 32-key blocks per tile
  static constexpr int NCB = D / 32;                       // 32-column blocks of O^T
  static constexpr int NKC = D / 16;                       // 16-wide QK^T k-chunks
  static constexpr int NT = BN / 16;                       // 16-key PV k-chunks
  static_assert(KG * (D / 8) == kThreads, "one V unit per thread");
  static_assert(K_CHUNKS * kThreads * 8 == BN * D, "K chunks cover the tile");
};

// Rows of the online softmax are rescaled only when their maximum grows by
// more than this many powers of two; otherwise exponentials are taken
// against the stale maximum and stay <= 2^8, which fp16 P and the fp32
// accumulators hold exactly as well. The final O / l and LSE use the same
// reference, so the result is the same in exact arithmetic.
constexpr float kRescaleLog2 = 8.0f;

// Position of key 4*kg (within the tile) in a V^T row. Keys
// 16t + 8h + 4g + q (h, g in {0,1}, q in 0..3) go to 16t + 8g + 4h + q, so the
// eight keys lane group g feeds to the t-th P.V instruction are contiguous.
__device__ __forceinline__ int vt_pos4(int kg) {
  return 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1);
}

// Global -> registers for the K tile starting at key n0 (keys >= N read 0).
template <int D>
__device__ __forceinline__ void load_k16(u32x4 *rk, const uint16_t *Kh, int n0, int N, int tid) {
  using S = Shape16<D>;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int c = 0; c < S::K_CHUNKS; ++c) {
    const int chunk = tid + c * kThreads;
    const int row = chunk / CPR, col8 = chunk % CPR;
    const int key = n0 + row;
    rk[c] = key < N ? *reinterpret_cast<const u32x4 *>(Kh + (size_t)key * D + col8 * 8)
                    : u32x4{0u, 0u, 0u, 0u};
  }
}

// Global -> registers for the V tile at n0: thread (kg = tid % KG,
// cg = tid / KG) holds keys 4kg..4kg+3 of columns 8cg..8cg+7, so the lanes
// sharing cg later write one V^T row together.
template <int D>
__device__ __forceinline__ void load_v16(u32x4 *rv, const uint16_t *Vh, int n0, int N, int tid) {
  using S = Shape16<D>;
  const int kg = tid % S::KG, cg = tid / S::KG;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int key = n0 + kg * 4 + q;
    rv[q] = key < N ? *reinterpret_cast<const u32x4 *>(Vh + (size_t)key * D + cg * 8)
                    : u32x4{0u, 0u, 0u, 0u};
  }
}

// Registers -> K stage: chunk c of this thread (row-major, padded rows).
template <int D>
__device__ __forceinline__ void store_k16_chunk(const u32x4 *rk, uint16_t *lk, int tid, int c) {
  using S = Shape16<D>;
  constexpr int CPR = D / 8;
  const int chunk = tid + c * kThreads;
  const int row = chunk / CPR, col8 = chunk % CPR;
  *reinterpret_cast<u32x4 *>(lk + row * S::KSTR + col8 * 8) = rk[c];
}

template <int D>
__device__ __forceinline__ void store_k16(const u32x4 *rk, uint16_t *lk, int tid) {
#pragma unroll
  for (int c = 0; c < Shape16<D>::K_CHUNKS; ++c) store_k16_chunk<D>(rk, lk, tid, c);
}

// V unit -> V^T (fp16), part w of 4: columns 8cg+2w and 8cg+2w+1, four keys
// each. Lanes with equal cg fill one V^T row, so the writes are free of bank
// conflicts.
template <int D, bool IS_BF16>
__device__ __forceinline__ void store_v16_part(const u32x4 *rv, uint16_t *lv, int tid, int w) {
  using S = Shape16<D>;
  const int kg = tid % S::KG, cg = tid / S::KG;
  uint16_t *dst = lv + (cg * 8) * S::VSTR + vt_pos4(kg);
  uint32_t lo0, lo1, hi0, hi1;  // (keys 0,1) and (keys 2,3) for columns 2w and 2w+1
  if (IS_BF16) {
    lo0 = pack_f16(bf16_lo_to_f32(rv[0][w]), bf16_lo_to_f32(rv[1][w]));
    hi0 = pack_f16(bf16_lo_to_f32(rv[2][w]), bf16_lo_to_f32(rv[3][w]));
    lo1 = pack_f16(bf16_hi_to_f32(rv[0][w]), bf16_hi_to_f32(rv[1][w]));
    hi1 = pack_f16(bf16_hi_to_f32(rv[2][w]), bf16_hi_to_f32(rv[3][w]));
  } else {
    lo0 = __builtin_amdgcn_perm(rv[1][w], rv[0][w], 0x05040100u);
    hi0 = __builtin_amdgcn_perm(rv[3][w], rv[2][w], 0x05040100u);
    lo1 = __builtin_amdgcn_perm(rv[1][w], rv[0][w], 0x07060302u);
    hi1 = __builtin_amdgcn_perm(rv[3][w], rv[2][w], 0x07060302u);
  }
  *reinterpret_cast<u32x2 *>(dst + (2 * w) * S::VSTR) = u32x2{lo0, hi0};
  *reinterpret_cast<u32x2 *>(dst + (2 * w + 1) * S::VSTR) = u32x2{lo1, hi1};
}

template <int D, bool IS_BF16>
__device__ __forceinline__ void store_v16(const u32x4 *rv, uint16_t *lv, int tid) {
#pragma unroll
  for (int w = 0; w < 4; ++w) store_v16_part<D, IS_BF16>(rv, lv, tid, w);
}

template <bool IS_BF16>
__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (IS_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_pv(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// S^T[kb] = K_kb Q^T for one tile: lane holds its query row and keys
// 32kb + 8(r/4) + 4g + r%4 of the tile. The two 32-key blocks are
// independent accumulation chains and are interleaved.
template <int D, bool IS_BF16>
__device__ __forceinline__ void qk_tile(f32x16 *s, const u32x4 *qf, const uint16_t *lk, int l32,
                                        int g) {
  using S = Shape16<D>;
#pragma unroll
  for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
  for (int kc = 0; kc < S::NKC; ++kc)
#pragma unroll
    for (int kb = 0; kb < S::NKB; ++kb) {
      const u32x4 a =
          *reinterpret_cast<const u32x4 *>(lk + (kb * 32 + l32) * S::KSTR + kc * 16 + g * 8);
      s[kb] = mfma_qk<IS_BF16>(a, qf[kc], s[kb]);
    }
}

// Per-lane online-softmax state: one query row, half of each tile's keys.
template <int D>
struct RowState16 {
  f32x16 acc[D / 32];  // O^T columns of this row (unnormalised)
  float m;             // reference maximum, base-2 units; -inf before any key
  float neg_m;         // -m, or 0 while m = -inf
  float l;             // sum of this lane's rounded weights
};

// Online-softmax update for one tile of scores, first half: mask (boundary
// tiles only), row maximum, lazy rescale of the state.
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void softmax_max(RowState16<D> &st, f32x16 *s, int n0, int N, int qrow,
                                            float qk, int g) {
  using S = Shape16<D>;
  if constexpr (MASK) {  // key tail and/or causal diagonal: hidden keys get -inf
#pragma unroll
    for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = n0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool dead = key >= N || (CAUSAL && key > qrow);
        s[kb][r] = dead ? -INFINITY : s[kb][r];
      }
  }
  // Row maximum of the scaled scores (qk > 0, so it is max(s) * qk).
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = fmaxf(mx, shfl_xor32(mx));
  const float m_tile = mx * qk;
  if (__any(m_tile > st.m + kRescaleLog2)) {  // wave-uniform: some row grew a lot
    const float m_new = fmaxf(st.m, m_tile);
    const float neg_new = m_new == -INFINITY ? 0.f : -m_new;
    const float alpha = exp2_fast(st.m + neg_new);  // 0 when m was -inf
#pragma unroll
    for (int cb = 0; cb < S::NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[cb][r] *= alpha;
    st.l *= alpha;
    st.m = m_new;
    st.neg_m = neg_new;
  }
}

// One packed P^T dword: weights p = 2^(s*qk - m) of two consecutive score
// registers rounded to fp16, and their (rounded) sum added to *lsum.
__device__ __forceinline__ uint32_t exp_pair(float s0, float s1, float qk, float neg_m,
                                             float *lsum) {
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  const float p0 = exp2_fast(fmaf(s0, qk, neg_m));
  const float p1 = exp2_fast(fmaf(s1, qk, neg_m));
  const uint32_t h = pack_f16(p0, p1);
  *lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h), ones, *lsum, false);
  return h;
}

// Everything one workgroup iteration touches.
template <int D>
struct Pipe16 {
  uint16_t *lds;      // K stage s at lds + s*K_ELEMS, V^T stages after both K stages
  const uint16_t *Kh, *Vh;
  u32x4 rk[Shape16<D>::K_CHUNKS];  // K tile j+2 in flight
  u32x4 rv[4];                     // V tile j+1 in flight
  f32x16 s[Shape16<D>::NKB];       // scores of the tile being normalised
  int N, n_tiles, qrow, tid, l32, g;
  float qk;
};

// LDS reads run this many MFMA steps ahead of their use.
constexpr int kLookahead = 3;

// Iteration j of the software pipeline. On entry: K_{j+1} and V_j are in
// LDS, S_j is in registers.
//  phase 0: row maxima of S_j and the (rare) rescale of the state;
//  phase 1: QK^T of tile j+1 on the matrix cores, one MFMA per step, each
//           step also computing two weights of tile j on the vector ALUs;
//  phase 2: P_j V_j, one MFMA per step, the first steps also writing the
//           prefetched V_{j+1} / K_{j+2} into the LDS stages freed last
//           iteration.
// Within a phase the vector work of a step does not depend on the MFMA in
// flight, so the two units run concurrently; scheduling barriers keep the
// compiler from regrouping the steps. NEXT = false for the last tile.
template <int D, bool IS_BF16, bool CAUSAL, bool MASK, bool NEXT>
__device__ __forceinline__ void pipe_iter(Pipe16<D> &pp, RowState16<D> &st, const u32x4 *qf, int j) {
  using S = Shape16<D>;
  constexpr int BN = S::BN;
  constexpr int LA = kLookahead;
  const bool k_next2 = NEXT && j + 2 < pp.n_tiles;
  const int l32 = pp.l32, g = pp.g;
  // Stage offsets are selected as integers so the pointers stay in LDS.
  uint16_t *const k_this = pp.lds + (j & 1) * S::K_ELEMS;
  uint16_t *const k_next = pp.lds + ((j + 1) & 1) * S::K_ELEMS;
  uint16_t *const v_this = pp.lds + 2 * S::K_ELEMS + (j & 1) * S::V_ELEMS;
  uint16_t *const v_next = pp.lds + 2 * S::K_ELEMS + ((j + 1) & 1) * S::V_ELEMS;
  if (NEXT) {
    if (k_next2) load_k16<D>(pp.rk, pp.Kh, (j + 2) * BN, pp.N, pp.tid);
    load_v16<D>(pp.rv, pp.Vh, (j + 1) * BN, pp.N, pp.tid);
  }

  // ---- phase 0
  softmax_max<D, CAUSAL, MASK>(st, pp.s, j * BN, pp.N, pp.qrow, pp.qk, g);

  // ---- phase 1: MFMA step i accumulates s_next[kb] += K_kb,kc Q_kc^T with
  // kc = i / NKB, kb = i % NKB (alternating accumulators), and packs the
  // next PPS P^T dwords of tile j.
  constexpr int NM1 = S::NKB * S::NKC;
  constexpr int PPS = S::NT * 4 / NM1;  // P^T dwords per step (1 for d=128, 2 for d=64)
  static_assert(PPS * NM1 == S::NT * 4, "P^T dwords split evenly over the QK^T MFMAs");
  f32x16 s_next[S::NKB];
  u32x4 pf[S::NT];
  float lsum = 0.f;
  const float qk = pp.qk, neg_m = st.neg_m;
  u32x4 kf[LA + 1];
  const uint16_t *kbase = k_next + l32 * S::KSTR + g * 8;
  if (NEXT) {
#pragma unroll
    for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_next[kb][r] = 0.f;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      kf[i] = *reinterpret_cast<const u32x4 *>(kbase + (i % S::NKB) * 32 * S::KSTR +
                                               (i / S::NKB) * 16);
  }
#pragma unroll
  for (int i = 0; i < NM1; ++i) {
    if (NEXT) {
      const int ia = i + LA;
      if (ia < NM1)
        kf[ia % (LA + 1)] = *reinterpret_cast<const u32x4 *>(
            kbase + (ia % S::NKB) * 32 * S::KSTR + (ia / S::NKB) * 16);
      const int kb = i % S::NKB, kc = i / S::NKB;
      s_next[kb] = mfma_qk<IS_BF16>(kf[i % (LA + 1)], qf[kc], s_next[kb]);
    }
#pragma unroll
    for (int q = 0; q < PPS; ++q) {
      const int dw = i * PPS + q, t = dw >> 2, w = dw & 3;
      const int kb = t >> 1, r = 8 * (t & 1) + 2 * w;
      pf[t][w] = exp_pair(pp.s[kb][r], pp.s[kb][r + 1], qk, neg_m, &lsum);
      asm volatile("" ::"v"(pf[t][w]));  // keep this step's weights in this step
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  st.l += lsum;

  // ---- phase 2: MFMA step i accumulates acc[cb] += V^T_cb,t P^T_t with
  // t = i / NCB, cb = i % NCB.
  constexpr int NM2 = S::NT * S::NCB;
  u32x4 vf[LA + 1];
  const uint16_t *vbase = v_this + l32 * S::VSTR + 8 * g;
#pragma unroll
  for (int i = 0; i < LA; ++i)
    vf[i] = *reinterpret_cast<const u32x4 *>(vbase + (i % S::NCB) * 32 * S::VSTR +
                                             16 * (i / S::NCB));
#pragma unroll
  for (int i = 0; i < NM2; ++i) {
    const int ia = i + LA;
    if (ia < NM2)
      vf[ia % (LA + 1)] = *reinterpret_cast<const u32x4 *>(
          vbase + (ia % S::NCB) * 32 * S::VSTR + 16 * (ia / S::NCB));
    const int cb = i % S::NCB, t = i / S::NCB;
    st.acc[cb] = mfma_pv(vf[i % (LA + 1)], pf[t], st.acc[cb]);
    if (NEXT) {
      if (i < 4) store_v16_part<D, IS_BF16>(pp.rv, v_next, pp.tid, i);
      if (i >= 4 && i < 4 + S::K_CHUNKS && k_next2)
        store_k16_chunk<D>(pp.rk, k_this, pp.tid, i - 4);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (NEXT) {
#pragma unroll
    for (int kb = 0; kb < S::NKB; ++kb) pp.s[kb] = s_next[kb];
    __syncthreads();
  }
}

template <int D, bool IS_BF16, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_16(FwdParams p) {
  using S = Shape16<D>;
  constexpr int BN = S::BN;
  constexpr int NCB = S::NCB;
  constexpr int NKC = S::NKC;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * S::K_ELEMS + 2 * S::V_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  int bh, qt;
  work_item<CAUSAL>(p, bh, qt);
  const int N = p.N;
  const int m0 = qt * kBlockM;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t *Qh = static_cast<const uint16_t *>(p.q) + head;

  Pipe16<D> pp;
  pp.lds = lds;
  pp.Kh = static_cast<const uint16_t *>(p.k) + head;
  pp.Vh = static_cast<const uint16_t *>(p.v) + head;
  pp.N = N;
  pp.tid = tid;
  pp.l32 = l32;
  pp.g = g;
  pp.qk = p.qk;
  // This lane's query row; rows past N read as zero and are never stored.
  pp.qrow = m0 + wave * 32 + l32;

  u32x4 qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    qf[kc] = pp.qrow < N
                 ? *reinterpret_cast<const u32x4 *>(Qh + (size_t)pp.qrow * D + kc * 16 + g * 8)
                 : u32x4{0u, 0u, 0u, 0u};

  // KV tiles to visit. Causal: only tiles holding some key <= the block's
  // last row. Tiles [0, n_full) need no mask at all.
  const int n_all = (N + BN - 1) / BN;
  const int n_tiles = CAUSAL ? min(n_all, (m0 + kBlockM + BN - 1) / BN) : n_all;
  int n_full = N / BN;
  if (CAUSAL) n_full = min(n_full, (m0 + 1) / BN);
  pp.n_tiles = n_tiles;

  RowState16<D> st;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[cb][r] = 0.f;
  st.m = -INFINITY;
  st.neg_m = 0.f;
  st.l = 0.f;

  // Prologue: K_0, V_0 and K_1 into LDS, then S_0.
  load_k16<D>(pp.rk, pp.Kh, 0, N, tid);
  load_v16<D>(pp.rv, pp.Vh, 0, N, tid);
  store_k16<D>(pp.rk, lds, tid);
  store_v16<D, IS_BF16>(pp.rv, lds + 2 * S::K_ELEMS, tid);
  if (n_tiles > 1) {
    load_k16<D>(pp.rk, pp.Kh, BN, N, tid);
    store_k16<D>(pp.rk, lds + S::K_ELEMS, tid);
  }
  __syncthreads();
  qk_tile<D, IS_BF16>(pp.s, qf, lds, l32, g);

  int j = 0;
  const int n_pipe = min(n_full, n_tiles - 1);  // unmasked tiles with a successor
  for (; j < n_pipe; ++j) pipe_iter<D, IS_BF16, CAUSAL, false, true>(pp, st, qf, j);
  for (; j < n_tiles - 1; ++j) pipe_iter<D, IS_BF16, CAUSAL, true, true>(pp, st, qf, j);
  if (j < n_full)
    pipe_iter<D, IS_BF16, CAUSAL, false, false>(pp, st, qf, j);
  else
    pipe_iter<D, IS_BF16, CAUSAL, true, false>(pp, st, qf, j);

  // Epilogue: combine the two key halves of the row sum, divide once, LSE.
  const float l_tot = st.l + shfl_xor32(st.l);
  const float l_safe = l_tot > 0.f ? l_tot : 1.f;
  const float inv = 1.0f / l_safe;
  const int qrow = pp.qrow;
  if (qrow < N) {
    if (g == 0) p.lse[(size_t)bh * N + qrow] = (st.m + log2_fast(l_safe)) * 0.69314718055994531f;
    const size_t orow = head + (size_t)qrow * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c0 = cb * 32 + r4 * 8 + g * 4;
        const float o0 = st.acc[cb][4 * r4 + 0] * inv, o1 = st.acc[cb][4 * r4 + 1] * inv;
        const float o2 = st.acc[cb][4 * r4 + 2] * inv, o3 = st.acc[cb][4 * r4 + 3] * inv;
        if (OUT_F32) {
          *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + orow + c0) = f32x4{o0, o1, o2, o3};
        } else if (IS_BF16) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const bf16x4 h = {(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3};
          *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(p.o) + orow + c0) = h;
        } else {
          typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
          const f16x4 h = {(_Float16)o0, (_Float16)o1, (_Float16)o2, (_Float16)o3};
          *reinterpret_cast<f16x4 *>(static_cast<uint16_t *>(p.o) + orow + c0) = h;
        }
      }
  }
}

// --------------------------------------------------------------------------
// fp32 kernel (v_mfma_f32_32x32x2_f32): same decomposition, 32-key tiles,
// single-buffered. A 32x32x2 step takes one value per lane, so V can stay
// row-major in LDS.
// --------------------------------------------------------------------------
template <int D>
struct Shape32 {
  static constexpr int BN = 32;
  static constexpr int KSTR = D + 2;  // conflict-free column reads of K
  static constexpr int VSTR = D + 8;  // rows 4 apart land 32 banks apart
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_f32(FwdParams p) {
  using S = Shape32<D>;
  constexpr int BN = S::BN;
  constexpr int NCB = D / 32;
  __shared__ float lk[BN * S::KSTR];
  __shared__ float lv[BN * S::VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  int bh, qt;
  work_item<CAUSAL>(p, bh, qt);
  const int N = p.N;
  const int m0 = qt * kBlockM;
  const size_t head = (size_t)bh * (size_t)N * D;
  const float *Qh = static_cast<const float *>(p.q) + head;
  const float *Kh = static_cast<const float *>(p.k) + head;
  const float *Vh = static_cast<const float *>(p.v) + head;

  const int qrow = m0 + wave * 32 + l32;
  float qf[D / 2];  // Q[qrow][2kk + g]
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) qf[kk] = qrow < N ? Qh[(size_t)qrow * D + 2 * kk + g] : 0.f;

  const int n_all = (N + BN - 1) / BN;
  const int n_tiles = CAUSAL ? min(n_all, (m0 + kBlockM + BN - 1) / BN) : n_all;

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  float m_i = -INFINITY, l_i = 0.f;
  const float qk = p.qk;

  for (int j = 0; j < n_tiles; ++j) {
    const int n0 = j * BN;
    __syncthreads();  // previous tile fully consumed
    for (int e = tid; e < BN * D; e += kThreads) {
      const int row = e / D, col = e % D;
      const int key = n0 + row;
      lk[row * S::KSTR + col] = key < N ? Kh[(size_t)key * D + col] : 0.f;
      lv[row * S::VSTR + col] = key < N ? Vh[(size_t)key * D + col] : 0.f;
    }
    __syncthreads();

    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(lk[l32 * S::KSTR + 2 * kk + g], qf[kk], s, 0, 0, 0);

    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = n0 + 8 * (r >> 2) + 4 * g + (r & 3);
      const bool dead = key >= N || (CAUSAL && key > qrow);
      s[r] = dead ? -INFINITY : s[r];
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, shfl_xor32(mx));
    const float m_new = fmaxf(m_i, mx * qk);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2_fast(m_i - m_use);
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2_fast(fmaf(s[r], qk, -m_use));
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
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(lv[key * S::VSTR + cb * 32 + l32], s[r],
                                                       acc[cb], 0, 0, 0);
      }
    }
  }

  const float l_tot = l_i + shfl_xor32(l_i);
  const float l_safe = l_tot > 0.f ? l_tot : 1.f;
  const float inv = 1.0f / l_safe;
  if (qrow < N) {
    if (g == 0) p.lse[(size_t)bh * N + qrow] = (m_i + log2_fast(l_safe)) * 0.69314718055994531f;
    float *orow = static_cast<float *>(p.o) + head + (size_t)qrow * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c0 = cb * 32 + r4 * 8 + g * 4;
        *reinterpret_cast<f32x4 *>(orow + c0) =
            f32x4{acc[cb][4 * r4] * inv, acc[cb][4 * r4 + 1] * inv, acc[cb][4 * r4 + 2] * inv,
                  acc[cb][4 * r4 + 3] * inv};
      }
  }
}

// --------------------------------------------------------------------------
// Host side: validation, dispatch, launch.
// --------------------------------------------------------------------------
typedef void (*KernelFn)(FwdParams);

template <int D, bool IS_BF16, bool CAUSAL>
KernelFn pick16(bool out_f32) {
  return out_f32 ? attn_fwd_16<D, IS_BF16, CAUSAL, true> : attn_fwd_16<D, IS_BF16, CAUSAL, false>;
}

template <int D>
KernelFn pick_d(attn_dtype in, bool out_f32, bool causal) {
  if (in == ATTN_F32) return causal ? attn_fwd_f32<D, true> : attn_fwd_f32<D, false>;
  if (in == ATTN_BF16) return causal ? pick16<D, true, true>(out_f32) : pick16<D, true, false>(out_f32);
  return causal ? pick16<D, false, true>(out_f32) : pick16<D, false, false>(out_f32);
}

thread_local int g_last_hip_error = 0;

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

int attn_last_hip_error(void) { return g_last_hip_error; }

const char *attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H or N out of range";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension or dtype combination";
    case ATTN_ERR_SCALE: return "scale must be finite and >= 0";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

attn_status attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                     int64_t H, int64_t N, int64_t d, int causal, float scale, attn_dtype in_dtype,
                     attn_dtype out_dtype, void *stream) {
  // Validation first: no HIP call happens before every argument is checked.
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if (N > (int64_t(1) << 24) || B * H > (int64_t(1) << 24)) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const bool in_ok = in_dtype == ATTN_F32 || in_dtype == ATTN_F16 || in_dtype == ATTN_BF16;
  if (!in_ok) return ATTN_ERR_UNSUPPORTED;
  if (in_dtype == ATTN_F32 && out_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (in_dtype != ATTN_F32 && out_dtype != in_dtype && out_dtype != ATTN_F32)
    return ATTN_ERR_UNSUPPORTED;
  if (!(scale >= 0.f) || !isfinite(scale)) return ATTN_ERR_SCALE;
  // Query rows per workgroup and threads per workgroup of the chosen kernel.
  const bool f32_path = in_dtype == ATTN_F32;
  const int64_t block_m = f32_path ? kBlockM : kBlockM16;
  const unsigned threads = f32_path ? kThreads : kThreads16;
  const int64_t nq = (N + block_m - 1) / block_m;
  const int64_t grid = nq * B * H;
  if (grid > INT32_MAX) return ATTN_ERR_SHAPE;

  FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.N = (int)N;
  p.nq = (int)nq;
  p.BH = (int)(B * H);
  // scale * log2(e) in double, rounded once; a zero scale becomes FLT_MIN so
  // masked scores (-inf) never meet a 0 factor.
  double qk = (double)scale * 1.4426950408889634;
  p.qk = qk < (double)FLT_MIN ? FLT_MIN : (float)qk;

  const bool out_f32 = out_dtype == ATTN_F32;
  KernelFn fn = d == 64 ? pick_d<64>(in_dtype, out_f32, causal != 0)
                        : pick_d<128>(in_dtype, out_f32, causal != 0);
  void *args[] = {&p};
  const hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((unsigned)grid),
                                         dim3(threads), args, 0, (hipStream_t)stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // extern "C"
