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
//  * each wave owns 32 query rows; a workgroup is 8 waves (256 rows, one
//    per CU) or 4 waves (128 rows), and the K/V tile 32 to 128 keys: two
//    tile shapes per head dimension are compiled, and the host picks one per
//    problem (pick_launch16).
//  * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16}: with the 32x32 output
//    layout each lane then holds the scores of ONE query row (lane & 31) for
//    16 keys per 32-key block, so the row maximum is an in-lane max plus one
//    exchange with lane ^ 32, and the row sum needs no exchange until the
//    end.
//  * O^T += V^T P^T on v_mfma_f32_32x32x16_f16: the B operand P^T comes
//    straight from the S^T accumulators of the same lane (converted to
//    fp16), and the O^T accumulator has the same row-per-lane layout, so
//    rescaling by alpha is a per-lane scalar multiply.
//  * K and V tiles are copied from memory straight into LDS rings
//    (buffer_load ... lds) and read from there by all the waves: K as the
//    A operand of QK^T, V through transposing reads (ds_read_b64_tr_b16)
//    as the A operand of O^T. bf16 V is converted to fp16 in place in LDS.
//  * each iteration is one stream of MFMAs (QK^T of the next tile, then P.V
//    of this one) with the softmax work spread across it: with operands read
//    from LDS and vector work between the MFMAs, two waves per SIMD that
//    each mix MFMAs with their own vector work keep the pipe busiest.
//  * a second instance of each bf16/fp16 kernel reads and writes through the
//    tensors' (batch, head, row) strides, with Nq query rows against Nk keys
//    and head dims below 64 or 128 read as zero columns (attn_fwd_strided);
//    the contiguous instance keeps those as compile-time constants.
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
  const void *v;     // V as the kernel reads it (the fp16 copy when a first pass made one)
  const void *v_in;  // V as the caller passed it
  void *o;
  float *lse;        // [B][H][N] contiguous
  // Element strides of (batch, head, row) of each tensor (columns are
  // unit-stride); vs for v, vis for v_in. The fp32 kernel takes contiguous
  // tensors only.
  int64_t qs[3], ks[3], vs[3], vis[3], os[3];
  int d;         // head dimension of the tensors: D, or (strided instances) a multiple of 8
                 // below it, whose columns d .. D-1 read as zeros and are not stored
  int N;         // sequence length (query rows per head)
  int Nk;        // keys per head: N, except for cross-attention (strided instances only)
  int nq;        // query tiles per (batch, head)
  int BH;        // batch * heads
  int H;         // heads
  float qk;      // scale * log2(e), >= FLT_MIN
};

// Element offset of head bh = b * H + h in a tensor with strides st.
__device__ __forceinline__ int64_t head_off(const int64_t *st, int bh, int H) {
  const int b = bh / H;
  return (int64_t)b * st[0] + (int64_t)(bh - b * H) * st[1];
}

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

// max / sum of x over lanes l and l ^ 32, without an LDS round trip:
// v_permlane32_swap exchanges the upper half of one register with the lower
// half of another, so swapping x with itself leaves {x[l], x[l ^ 32]} in the
// two results of every lane.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// --------------------------------------------------------------------------
// bf16 / fp16 kernel
// --------------------------------------------------------------------------
// Each wave owns 32 query rows. For d=128 a workgroup is 8 waves (256 rows,
// one workgroup per CU, two of its waves per SIMD): every K/V tile copied
// into LDS, and every bf16 V tile converted there, then serves twice as many
// rows as with 4-wave workgroups, which measured 5-7% faster despite the
// two waves of a SIMD meeting at the same barriers. For d=64 (128-key
// tiles) a workgroup is 4 waves and two share a CU, which measured faster
// there. K and V tiles go from global memory straight into LDS
// (buffer_load ... lds, no register staging), each through a ring of two
// stages (fetched one iteration before use). Both stay row-major; 16-byte chunks are XOR-swizzled per row so
// the lane-contiguous DMA writes, the K operand reads and the transposing V
// reads (ds_read_b64_tr_b16) are free of bank conflicts or nearly so. bf16 V
// is converted to fp16 in place in LDS (the P.V product runs in fp16, see
// the header), each thread converting the bytes its own copy brought in.
// Tiles: d=128 uses 64 keys, d=64 uses 128.
//
// Each iteration is one stream of 2 x 16 MFMAs (QK^T of tile j+1, then
// P_j V_j) with the softmax work of the tile -- the exponentials of S_j and
// the row maximum of S_{j+1} -- spread over all of its steps: about four
// vector instructions per MFMA run in its shadow when the two waves sharing
// a SIMD both interleave this way.
constexpr int kKStages = 2;
constexpr int kVStages = 2;

// Tile shape: waves per workgroup (32 query rows each; 8 -> one workgroup of
// 256 rows per CU, 4 -> two of 128 rows) and keys per K/V tile, per head
// dimension. The defaults are the measured choices (io_aware_attention_flash_amd/
// sweep.py builds and times the alternatives); a build may override them
// with -D. Combinations whose LDS does not fit, or whose tile copy is not a
// whole number of instructions, fail to compile.
// A -D choice of a head dimension's tile applies to every problem; without
// one the library chooses between two tiles per problem (see pick_launch16).
#if defined(ATTN_CFG_FWD_WAVES_D64) || defined(ATTN_CFG_FWD_BN_D64)
#define ATTN_FWD_D64_FORCED 1
#else
#define ATTN_FWD_D64_FORCED 0
#endif
#if defined(ATTN_CFG_FWD_WAVES_D128) || defined(ATTN_CFG_FWD_BN_D128)
#define ATTN_FWD_D128_FORCED 1
#else
#define ATTN_FWD_D128_FORCED 0
#endif
#ifndef ATTN_CFG_FWD_WAVES_D128
#define ATTN_CFG_FWD_WAVES_D128 8
#endif
#ifndef ATTN_CFG_FWD_BN_D128
#define ATTN_CFG_FWD_BN_D128 64
#endif
#ifndef ATTN_CFG_FWD_WAVES_D64
#define ATTN_CFG_FWD_WAVES_D64 4
#endif
#ifndef ATTN_CFG_FWD_BN_D64
#define ATTN_CFG_FWD_BN_D64 128
#endif

template <int D_, int WAVES_, int BN_>
struct Shape16 {
  static constexpr int D = D_;
  static constexpr int WAVES = WAVES_;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BLOCK_M = WAVES * 32;             // query rows per workgroup
  static constexpr int WG_PER_CU = 8 / WAVES;            // two waves per SIMD
  static constexpr int BN = BN_;
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int TILE_ELEMS = BN * D;              // one K or V stage
  static constexpr int TILE_BYTES = TILE_ELEMS * 2;
  static constexpr int DMA_INS = BN * CPR / THREADS;     // DMA instructions per thread and tile
  static constexpr int INS_BYTES = THREADS * 16;         // bytes one DMA instruction moves
  static constexpr int Q_INS = BLOCK_M * D * 2 / INS_BYTES;  // DMA instructions for the Q tile
  static constexpr int RING_ELEMS = 4 * TILE_ELEMS;      // K stages 0..1, V stages 0..1
  static_assert(kKStages + kVStages == 4, "ring size");
  // A workgroup alone on its CU stages O for the epilogue in LDS of its own,
  // in 128-byte rows, so it can copy its next tile's first K/V tiles and Q
  // into the ring while it writes out O; two workgroups per CU have no room
  // for that and stage in the ring, in 256-byte rows.
  static constexpr bool OWN_STAGE = WG_PER_CU == 1;
  static constexpr int STAGE_ROWB = OWN_STAGE ? 128 : 256;
  static constexpr int STAGE_ELEMS = OWN_STAGE ? WAVES * 32 * STAGE_ROWB / 2 : 0;
  static constexpr int LDS_ELEMS = RING_ELEMS + BLOCK_M * D + STAGE_ELEMS;
  static constexpr int NKB = BN / 32;                    // 32-key blocks per tile
  static constexpr int NCB = D / 32;                     // 32-column blocks of O^T
  static constexpr int NKC = D / 16;                     // 16-wide QK^T k-chunks
  static constexpr int NT = BN / 16;                     // 16-key PV k-chunks
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves per workgroup");
  static_assert(BN == 32 || BN == 64 || BN == 128, "32, 64 or 128 keys per tile");
  static_assert(DMA_INS >= 1 && DMA_INS * THREADS == BN * CPR, "DMA covers the tile");
  static_assert(DMA_INS * INS_BYTES == TILE_BYTES, "each DMA instruction moves 16 bytes a thread");
  static_assert((INS_BYTES / (D * 2)) % 16 == 0, "one copy instruction spans whole swizzle periods");
  static_assert(WG_PER_CU * LDS_ELEMS * 2 <= 160 * 1024, "LDS of the workgroups sharing a CU");
  // epilogue staging fits (own area, or the ring)
  static_assert(WAVES * 32 * (OWN_STAGE ? 128 : 256) <= (OWN_STAGE ? STAGE_ELEMS : RING_ELEMS) * 2,
                "O staging fits");
};

// The default tile of each head dimension.
template <int D>
using Tile16 = Shape16<D, D == 128 ? ATTN_CFG_FWD_WAVES_D128 : ATTN_CFG_FWD_WAVES_D64,
                       D == 128 ? ATTN_CFG_FWD_BN_D128 : ATTN_CFG_FWD_BN_D64>;

// Compile-time configuration. The defaults are the measured choices; a build
// may override them with -D (io_aware_attention_flash_amd/sweep.py builds
// and times the alternatives).
#ifndef ATTN_CFG_RESCALE_LOG2
#define ATTN_CFG_RESCALE_LOG2 8
#endif
#ifndef ATTN_CFG_LOOKAHEAD
#define ATTN_CFG_LOOKAHEAD 3
#endif
#ifndef ATTN_CFG_PREPASS_MIN_N
#define ATTN_CFG_PREPASS_MIN_N 8192
#endif
// Order of the two causal query tiles a workgroup takes: 0 runs the long one
// first, 1 the short one (which then reads the keys the long one starts
// with while they are fresh in L2), 2 alternates: pairs with an odd index run
// the short tile first, the others the long one.
#ifndef ATTN_CFG_CAUSAL_SHORT_FIRST
#define ATTN_CFG_CAUSAL_SHORT_FIRST 0
#endif
// Copies of the query tile with the non-temporal hint (1; each query row is
// read once) or plain (0).
#ifndef ATTN_CFG_Q_NONTEMPORAL
#define ATTN_CFG_Q_NONTEMPORAL 0
#endif
// Heads of one XCD when B*H is a multiple of 8: every eighth head (0: XCD x
// runs heads x, x+8, ...) or a block of B*H/8 adjacent ones (1).
#ifndef ATTN_CFG_HEAD_BLOCKED
#define ATTN_CFG_HEAD_BLOCKED 0
#endif
// Causal workgroups take a pair of query tiles (long + short, 1) or one
// tile each, longest first (0).
#ifndef ATTN_CFG_CAUSAL_PAIRS
#define ATTN_CFG_CAUSAL_PAIRS 1
#endif
// Stores of O with the non-temporal hint (streamed past L2 and the Infinity
// Cache, which then keep more of the K/V tiles the workgroups re-read) or
// plain. The epilogue writes whole 128-byte lines; the hint measured +2.5% to
// +3.8% at the causal N=4096 d=128 workload.
#ifndef ATTN_CFG_O_NONTEMPORAL
#define ATTN_CFG_O_NONTEMPORAL 1
#endif

// Rows of the online softmax are rescaled only when their maximum grows by
// more than this many powers of two; otherwise exponentials are taken
// against the stale maximum and stay <= 2^8 (at the default), which fp16 P
// and the fp32 accumulators hold exactly as well. The final O / l and LSE
// use the same reference, so the result is the same in exact arithmetic.
constexpr float kRescaleLog2 = ATTN_CFG_RESCALE_LOG2;
static_assert(ATTN_CFG_RESCALE_LOG2 >= 0 && ATTN_CFG_RESCALE_LOG2 <= 15, "fp16 P holds up to 2^15");

// LDS operand reads run this many MFMA steps ahead of their use.
constexpr int kLookahead = ATTN_CFG_LOOKAHEAD;
static_assert(kLookahead >= 1 && kLookahead <= 6, "lookahead range");

// Chunk swizzles: chunk x of row r is stored at x ^ swz(r).
//  K: the 16 rows one K operand read touches (same logical chunk) land on 16
//     different bank groups.
//  V: the 4 rows x 4 chunks of one transposing read land on each bank at
//     most twice.
// Both only depend on the row modulo 16, so they repeat within the 16 (d=128)
// or 32 (d=64) rows one DMA instruction covers.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// LDS byte address of a __shared__ element.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t *)p;
}

// Word 3 of a raw (untyped, stride 0) buffer descriptor on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;

// Buffer descriptor (four SGPR words) of tile t (keys t*BN ..) of one
// head's K or V with rows rs elements apart, cut to the keys that exist
// (empty for tiles past the last one visited), so reads beyond the cut
// return zeros and touch no memory. Every input is wave-uniform;
// readfirstlane says so to the compiler, which keeps the words in scalar
// registers.
template <class S>
__device__ __forceinline__ u32x4 tile_rsrc(const uint16_t *head, int t, int n_tiles, int N, int rs,
                                           int dcol) {
  constexpr int BN = S::BN;
  const int keys = t < n_tiles ? min(N - t * BN, BN) : 0;
  const uint16_t *base = keys > 0 ? head + (size_t)t * BN * (size_t)rs : head;
  // the last key's row ends dcol elements after its start: (keys - 1) rows
  // of rs elements and one of dcol (keys * D * 2 bytes for contiguous rows);
  // rows at or past `keys` start at or past that end (rs >= dcol)
  const uint32_t bytes = (uint32_t)(keys * rs * 2 - (keys > 0 ? (rs - dcol) * 2 : 0));
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xFFFFu,  // stride 0
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), (uint32_t)kBufferFlags};
}

// One buffer_load_dwordx4 ... lds: 16 bytes per lane from the descriptor at
// the lane's offset into LDS at lds_byte + 16 * lane. Written as inline
// assembly on purpose: the compiler then does not treat the copies in flight
// as possible writers of every LDS location, which would make it wait for
// all of them before each LDS read; this kernel orders them itself (an
// explicit vmcnt wait and a barrier before a stage is read, a barrier before
// it is refilled). M0 carries the LDS address; nothing else here uses it.
__device__ __forceinline__ void dma16_to_lds(u32x4 rsrc, uint32_t lds_byte, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_byte), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// The same with the non-temporal hint, for data read once (the query tile).
__device__ __forceinline__ void dma16_to_lds_nt(u32x4 rsrc, uint32_t lds_byte, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(lds_byte), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// DMA of one K or V tile into an LDS stage. Instruction c fills the 16-byte
// slots c*THREADS + tid: slot s holds physical chunk s % CPR of tile row
// s / CPR, i.e. logical chunk (s % CPR) ^ swz(row). Instruction c covers
// THREADS / CPR rows of the tile, a whole number of swizzle periods, so its
// lane offset is that of c = 0 plus c * (THREADS / CPR) rows of rs elements.
// The offset stays in a VGPR (the descriptor's range check applies to it,
// not to an SGPR offset).
// With PAD, a lane whose 16-byte piece starts at or past column dcol gets
// kOutOfRange instead: every copy of it reads zeros (the offsets of later
// instructions add less than 2^30 to it, so they stay out of range too).
constexpr uint32_t kOutOfRange = 0x80000000u;
template <int D, bool IS_V, bool PAD>
__device__ __forceinline__ uint32_t dma_offset(int tid, int rs, int dcol) {
  constexpr int CPR = D / 8;
  const int row0 = tid / CPR;
  const int swz = IS_V ? swz_v<D>(row0) : swz_k<D>(row0);
  const int lc = (tid % CPR) ^ swz;  // logical 16-byte chunk of the row
  if (PAD && lc * 8 >= dcol) return kOutOfRange;
  return (uint32_t)(row0 * rs * 2) + (lc << 4);
}
// Wait until at most N vector-memory instructions of this wave are
// outstanding (they retire in order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS writes of this wave done, then a workgroup barrier. (No memory fence:
// it would also wait for the copies in flight.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
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

// Lane-constant parts of the LDS operand addresses (elements).
template <int D>
struct LaneAddr {
  int k_off;          // K operand: row l32
  int k_swz;          // swz_k of this lane's rows, with g folded in
  int v_off[D / 32];  // V operand (transposing read), per 32-column block
};

template <int D>
__device__ __forceinline__ LaneAddr<D> lane_addr(int lane) {
  LaneAddr<D> la;
  const int l32 = lane & 31, g = lane >> 5;
  la.k_swz = swz_k<D>(l32) ^ g;  // logical chunk 2kc + g = 2kc ^ g
  la.k_off = l32 * D;
  // Transposing read, 16-lane block (g, h), source lane s = a + 4m: row
  // 4g + m (plus multiples of 8 rows), columns 32cb + 16h + 4a .. +3.
  const int s = lane & 15, h = (lane >> 4) & 1;
  const int a = s & 3, m = s >> 2;
  const int row = 4 * g + m;
  const int sv = swz_v<D>(row);
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
    const int x = 4 * cb + 2 * h + (a >> 1);
    la.v_off[cb] = row * D + (x ^ sv) * 8 + (a & 1) * 4;
  }
  return la;
}

// K operand of QK^T step (kb, kc): K[32kb + l32][16kc + 8g .. +7].
template <int D>
__device__ __forceinline__ u32x4 k_frag(const uint16_t *kst, const LaneAddr<D> &la, int kb,
                                        int kc) {
  return *reinterpret_cast<const u32x4 *>(kst + la.k_off + kb * 32 * D +
                                          (((2 * kc) ^ la.k_swz) << 3));
}

// V^T operand of PV step (t, cb): keys 16t + 8u + 4g + 0..3 (u = 0, 1) of
// column 32cb + l32, as 8 fp16 values -- the key order of the P^T operand
// taken from the S^T accumulators.
template <int D>
__device__ __forceinline__ u32x4 v_frag(const uint16_t *vst, const LaneAddr<D> &la, int t, int cb) {
  const uint16_t *p0 = vst + la.v_off[cb] + (16 * t) * D;
  const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p0));
  const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p0 + 8 * D));
  const u32x2 w0 = __builtin_bit_cast(u32x2, r0), w1 = __builtin_bit_cast(u32x2, r1);
  return u32x4{w0[0], w0[1], w1[0], w1[1]};
}

// S^T[kb] = K_kb Q^T for one tile (once per query tile, before the
// pipelined loop), the K operands read kLookahead steps ahead of their MFMAs.
template <class S, bool IS_BF16>
__device__ __forceinline__ void qk_tile(f32x16 *s, const u32x4 *qf, const uint16_t *kst,
                                        const LaneAddr<S::D> &la) {
  constexpr int D = S::D;
  constexpr int NM = S::NKB * S::NKC, LA = kLookahead;
  u32x4 fr[LA + 1];
#pragma unroll
  for (int i = 0; i < LA; ++i) fr[i] = k_frag<D>(kst, la, i / S::NKC, i % S::NKC);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    const int ia = i + LA;
    if (ia < NM) fr[ia % (LA + 1)] = k_frag<D>(kst, la, ia / S::NKC, ia % S::NKC);
    const int kb = i / S::NKC, kc = i % S::NKC;
    s[kb] = mfma_qk<IS_BF16>(fr[i % (LA + 1)], qf[kc], kc == 0 ? f32x16{} : s[kb]);
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

// Score register r of block kb belongs to key 32kb + 8(r/4) + 4g + r%4 of the
// tile (the 32x32 MFMA output layout); masked keys become -inf.
template <bool CAUSAL>
__device__ __forceinline__ float mask_score(float x, int key, int N, int qrow) {
  const bool dead = key >= N || (CAUSAL && key > qrow);
  return dead ? -INFINITY : x;
}
__device__ __forceinline__ int score_key(int n0, int kb, int r, int g) {
  return n0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
}

// New reference maximum from a tile's row maximum m_tile (base-2 units): the
// rare rescale of the state, taken by the whole wave when some row's maximum
// grew by more than kRescaleLog2.
template <int D>
__device__ __forceinline__ void rescale(RowState16<D> &st, float m_tile) {
  if (__any(m_tile > st.m + kRescaleLog2)) {
    const float m_new = fmaxf(st.m, m_tile);
    const float neg_new = m_new == -INFINITY ? 0.f : -m_new;
    const float alpha = exp2_fast(st.m + neg_new);  // 0 when m was -inf
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[cb][r] *= alpha;
    st.l *= alpha;
    st.m = m_new;
    st.neg_m = neg_new;
  }
}

// Mask, row maximum and rescale for a whole tile of scores at once (the
// first tile; later tiles do this inside phase 2).
template <class S, bool CAUSAL, bool MASK>
__device__ __forceinline__ void softmax_max(RowState16<S::D> &st, f32x16 *s, int n0, int N, int qrow,
                                            float qk, int g) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < S::NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (MASK) s[kb][r] = mask_score<CAUSAL>(s[kb][r], score_key(n0, kb, r, g), N, qrow);
      mx = fmaxf(mx, s[kb][r]);
    }
  rescale<S::D>(st, max_halves(mx) * qk);  // qk > 0: the max of the scaled scores
}

// Eight bf16 values -> eight fp16 values (round to nearest even; exact for
// |v| in [2^-14, 65504]).
__device__ __forceinline__ u32x4 to_f16(u32x4 x) {
  u32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = pack_f16(bf16_lo_to_f32(x[e]), bf16_hi_to_f32(x[e]));
  return y;
}

// Everything the iterations of one wave touch.
template <class S>
struct Pipe16 {
  static constexpr int D = S::D;
  uint16_t *lds;  // K stages 0..1, then V stages 0..1 (tile t in stage t % 2)
  const uint16_t *Kh, *Vh;
  LaneAddr<D> la;
  int N, Nq, n_tiles, qrow, g, tid;  // N: keys per head; Nq: query rows per head
  uint32_t lds_wave;  // LDS byte address of the buffer plus 1024 * wave (uniform)
  // Source offsets of this thread's 16 bytes in copy instruction c (kept in
  // registers: the descriptor's range check applies to them), and that of
  // the query tile's first copy instruction.
  uint32_t k_dma[S::DMA_INS], v_dma[S::DMA_INS], q_dma0;
  int qrs, krs, vrs;  // row strides (elements) of Q, K and V
  int dcol;           // columns of the tensors (D, or fewer for strided instances)
  float qk;

  __device__ __forceinline__ uint16_t *kstage(int par) const {
    return lds + par * S::TILE_ELEMS;
  }
  __device__ __forceinline__ uint16_t *vstage(int par) const {
    return lds + (kKStages + par) * S::TILE_ELEMS;
  }
  // The query tile (BLOCK_M rows, K's layout) after the rings.
  __device__ __forceinline__ uint16_t *qstage() const { return lds + S::RING_ELEMS; }
  // Tile copies. Iteration j reads K_{j+1} and V_j. Its first steps issue
  // V_{j+1}, then K_{j+2}, into the stages V_{j-1} and K_j left (free since
  // the barrier that ended iteration j-1); a late step waits for V_{j+1}
  // and converts it (bf16); the iteration ends by waiting for K_{j+2}.
  __device__ __forceinline__ u32x4 k_rsrc(int t) const {
    return tile_rsrc<S>(Kh, t, n_tiles, N, krs, dcol);
  }
  __device__ __forceinline__ u32x4 v_rsrc(int t) const {
    return tile_rsrc<S>(Vh, t, n_tiles, N, vrs, dcol);
  }
  // Instruction c of the copy of K_t / V_t (descriptor r).
  __device__ __forceinline__ void copy_k(u32x4 r, int t, int c) const {
    constexpr int TB = S::TILE_BYTES;
    dma16_to_lds(r, lds_wave + (t & 1) * TB + c * S::INS_BYTES, k_dma[c]);
  }
  __device__ __forceinline__ void copy_v(u32x4 r, int t, int c) const {
    constexpr int TB = S::TILE_BYTES;
    dma16_to_lds(r, lds_wave + (kKStages + (t & 1)) * TB + c * S::INS_BYTES, v_dma[c]);
  }
  // Copy of the workgroup's query tile (rows m0 ..; rows past Nq read as 0).
  __device__ __forceinline__ void issue_q(const uint16_t *Qh, int m0) const {
    const int rows = min(Nq - m0, S::BLOCK_M);
    const uint64_t a = reinterpret_cast<uint64_t>(Qh + (size_t)m0 * (size_t)qrs);
    const u32x4 r = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xFFFFu,
                     (uint32_t)__builtin_amdgcn_readfirstlane(((rows - 1) * qrs + dcol) * 2),
                     (uint32_t)kBufferFlags};
    constexpr int RPI = S::THREADS / S::CPR;  // rows per copy instruction
#pragma unroll
    for (int c = 0; c < S::Q_INS; ++c) {
      const uint32_t dst = lds_wave + S::RING_ELEMS * 2 + c * S::INS_BYTES;
      const uint32_t off = q_dma0 + (uint32_t)(c * RPI * qrs * 2);
      if (ATTN_CFG_Q_NONTEMPORAL)
        dma16_to_lds_nt(r, dst, off);
      else
        dma16_to_lds(r, dst, off);
    }
  }
  __device__ __forceinline__ void issue_k(int t) const {
    const u32x4 r = k_rsrc(t);
#pragma unroll
    for (int c = 0; c < S::DMA_INS; ++c) copy_k(r, t, c);
  }
  __device__ __forceinline__ void issue_v(int t) const {
    const u32x4 r = v_rsrc(t);
#pragma unroll
    for (int c = 0; c < S::DMA_INS; ++c) copy_v(r, t, c);
  }
  // 16-byte slot c of the ones this thread's own copy of V_t wrote: after
  // the copy has landed (this wave's vmcnt wait), the thread converts them
  // from bf16 to fp16 in place.
  __device__ __forceinline__ u32x4 *v_slot(int t, int c) const {
    return reinterpret_cast<u32x4 *>(vstage(t & 1) + c * (S::INS_BYTES / 2) + tid * 8);
  }
  template <bool CONV_V>
  __device__ __forceinline__ void convert_v(int t) const {
    if (!CONV_V || t >= n_tiles) return;
#pragma unroll
    for (int c = 0; c < S::DMA_INS; ++c) *v_slot(t, c) = to_f16(*v_slot(t, c));
  }
};

// Step at which score pair p (P^T dword p % 4 of PV operand p / 4, scores
// of block p / 8) takes its exponent argument; its exponential follows one
// step later and its fp16 pack and row sum one more later. The NM1 QK^T steps
// come first, then the NM2 P.V steps. The first F pairs are spread over the
// first FS steps, the rest over the steps left before their P.V steps: the
// QK^T steps finish the blocks of S_{j+1} from the last to the first, and
// taking S_j's first blocks early lets the later blocks of S_{j+1} reuse
// their registers (five blocks live at a time for d=128, six for d=64, not
// eight), while the vector work still spreads over most of the MFMAs.
template <class S>
struct PairPlan {
  static constexpr int D = S::D;
  static constexpr int NM1 = S::NKB * S::NKC;
  static constexpr int NM2 = S::NT * S::NCB;
  static constexpr int NP = S::NT * 4;
  static constexpr int deadline(int p) { return NM1 + (p >> 2) * S::NCB - 1; }
  static constexpr int LAST = deadline(NP - 1) - 2;
  static constexpr int start_fs(int p, int f, int fs) {
    return p < f ? p * fs / f : fs + (p - f) * (LAST - fs) / (NP - 1 - f);
  }
  static constexpr bool valid_fs(int f, int fs) {
    for (int p = 0; p < NP; ++p)
      if (start_fs(p, f, fs) + 2 > deadline(p) || (p > 0 && start_fs(p, f, fs) < start_fs(p - 1, f, fs)))
        return false;
    return start_fs(NP - 1, f, fs) == LAST;
  }
  // The measured spread for the default tiles (d=128: 64 keys, d=64: 128);
  // for other tiles the widest valid one, front pairs first.
  static constexpr int pick(bool want_fs) {
    if (D == 128 && S::BN == 64 && valid_fs(8, 8)) return 8;
    if (D == 64 && S::BN == 128 && valid_fs(16, 12)) return want_fs ? 12 : 16;
    for (int f = NP / 2; f >= 1; --f)
      for (int fs = f; fs >= 1; --fs)
        if (valid_fs(f, fs)) return want_fs ? fs : f;
    return 0;
  }
  static constexpr int F = pick(false);
  static constexpr int FS = pick(true);
  static constexpr int start(int p) { return start_fs(p, F, FS); }
  static_assert(F > 0 && valid_fs(F, FS), "every pair is packed before its P.V step");
  // First pair starting at step i or later, and the most pairs one step starts.
  static constexpr int first_at(int i) {
    int p = 0;
    while (p < NP && start(p) < i) ++p;
    return p;
  }
  static constexpr int max_per_step() {
    int m = 0;
    for (int i = 0; i <= LAST; ++i) m = first_at(i + 1) - first_at(i) > m ? first_at(i + 1) - first_at(i) : m;
    return m;
  }
  static constexpr int MAXP = max_per_step();
};

// Iteration j of one wave: on entry K_{j+1} and V_j are in LDS and S_j (s)
// is in registers, masked, its maximum folded into the reference. Steps
// 0..NM1-1: s_next[kb] += K_kb,kc Q_kc^T (NEXT; kb = NKB-1 - i / NKC,
// kc = i % NKC). Steps NM1..NM1+NM2-1: acc[cb] += V^T_cb,t P^T_t
// (t = i' / NCB, cb = i' % NCB). Alongside, on the vector ALUs: the
// weights of S_j (three stages per score pair, in successive steps, so no
// instruction waits on the one before) and, in the P.V steps, the mask
// (MASK_NEXT) and row maximum of S_{j+1}, blocks in the order they were
// finished. Then the (rare) rescale for S_{j+1}. Scheduling barriers keep
// the compiler from regrouping the steps. The first 2 DMA_INS steps also
// issue the copies of V_{j+1} and K_{j+2}, one instruction each; step CW
// waits for V_{j+1} and the steps after it convert it (bf16), one 16-byte
// slot per two steps (load, then convert and store). VPAR is j's parity
// when known at compile time (-1 otherwise), which makes the V stage
// addresses constants.
template <class S, bool IS_BF16, bool CONV_V, bool CAUSAL, bool MASK_NEXT, bool NEXT, int VPAR>
__device__ __forceinline__ void iteration(const Pipe16<S> &pp, RowState16<S::D> &st, const u32x4 *qf,
                                          int j, f32x16 (&s)[S::NKB], f32x16 (&s_next)[S::NKB]) {
  constexpr int D = S::D;
  using PP = PairPlan<S>;
  constexpr int LA = kLookahead;
  constexpr int NM1 = PP::NM1, NM2 = PP::NM2, NP = PP::NP;
  constexpr int NS = NM1 + NM2;
  constexpr int NE = S::NKB * 16;  // scores of S_{j+1} per lane
  static_assert(NE % NM2 == 0, "scores split evenly over the P.V steps");
  constexpr int EPS = NE / NM2;
  const uint16_t *k_next = pp.kstage(VPAR >= 0 ? 1 - VPAR : ((j + 1) & 1));
  const uint16_t *v_this = pp.vstage(VPAR >= 0 ? VPAR : (j & 1));
  const int n1 = (j + 1) * S::BN;
  u32x4 pf[S::NT];
  float xa[NP][2], ea[NP][2];  // exponent arguments, exponentials
  float lsum = 0.f, mx = -INFINITY;
  const float qk = pp.qk, neg_m = st.neg_m;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  // LDS operands run LA steps ahead; fr[i % (LA + 1)] holds step i's.
  u32x4 fr[LA + 1];
  constexpr int NI = S::DMA_INS;
  constexpr int CW = NS - 2 * NI - 2;  // conversion steps CW .. CW + 2 NI
  static_assert(CW >= 2 * NI, "V_{j+1} is converted after its copy was issued");
  u32x4 cv[NI];
  auto operand = [&](int i) -> u32x4 {
    if (i < NM1) return k_frag<D>(k_next, pp.la, S::NKB - 1 - i / S::NKC, i % S::NKC);
    const int i2 = i - NM1;
    return v_frag<D>(v_this, pp.la, i2 / S::NCB, i2 % S::NCB);
  };
  const int first = NEXT ? 0 : NM1;  // the last tile has no QK^T steps
  const u32x4 dv_r = pp.v_rsrc(j + 1), dk_r = pp.k_rsrc(j + 2);
#pragma unroll
  for (int i = 0; i < LA; ++i)
    if (first + i < NS) fr[(first + i) % (LA + 1)] = operand(first + i);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (i >= first) {
      const int ia = i + LA;
      if (ia < NS) fr[ia % (LA + 1)] = operand(ia);
      if (i < NM1) {
        const int kb = S::NKB - 1 - i / S::NKC, kc = i % S::NKC;
        s_next[kb] = mfma_qk<IS_BF16>(fr[i % (LA + 1)], qf[kc], kc == 0 ? f32x16{} : s_next[kb]);
      } else {
        const int i2 = i - NM1, cb = i2 % S::NCB, t = i2 / S::NCB;
        st.acc[cb] = mfma_pv(fr[i % (LA + 1)], pf[t], st.acc[cb]);
      }
    }
#pragma unroll
    for (int q = 0; q < PP::MAXP; ++q) {
      const int pa = PP::first_at(i) + q;  // exponent arguments
      if (pa < NP && PP::start(pa) == i) {
        const int t = pa >> 2, kb = t >> 1, r = 8 * (t & 1) + 2 * (pa & 3);
        xa[pa][0] = fmaf(s[kb][r], qk, neg_m);
        xa[pa][1] = fmaf(s[kb][r + 1], qk, neg_m);
      }
      const int pb = PP::first_at(i - 1) + q;  // exponentials
      if (i >= 1 && pb < NP && PP::start(pb) == i - 1) {
        ea[pb][0] = exp2_fast(xa[pb][0]);
        ea[pb][1] = exp2_fast(xa[pb][1]);
      }
      const int pc = PP::first_at(i - 2) + q;  // fp16 pack and row sum
      if (i >= 2 && pc < NP && PP::start(pc) == i - 2) {
        const uint32_t h = pack_f16(ea[pc][0], ea[pc][1]);
        lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h), ones, lsum, false);
        pf[pc >> 2][pc & 3] = h;
        // keep this pair's weights and its share of the row sum in this step
        asm volatile("" : "+v"(lsum) : "v"(h));
      }
    }
    if (CONV_V && i >= CW && i <= CW + 2 * NI) {
      // Slot c is read at step CW + 2c; its first two dwords are converted
      // one step later, the other two and the store one more later. Past
      // the last tile the copy brought zeros, which convert harmlessly.
      const int k = i - CW;
      if (k == 0) wait_vmcnt<NI>();  // V_{j+1} (issued before K_{j+2}) is in
      if ((k & 1) == 0 && k / 2 < NI) cv[k / 2] = *pp.v_slot(j + 1, k / 2);
      if (k >= 1) {
        const int c = (k - 1) >> 1, e0 = 2 * ((k - 1) & 1);
#pragma unroll
        for (int e = e0; e < e0 + 2; ++e) {
          cv[c][e] = pack_f16(bf16_lo_to_f32(cv[c][e]), bf16_hi_to_f32(cv[c][e]));
          asm volatile("" : "+v"(cv[c][e]));
        }
        if (e0 == 2) *pp.v_slot(j + 1, c) = cv[c];
      }
    }
    if (i < S::DMA_INS) pp.copy_v(dv_r, j + 1, i);
    if (i >= S::DMA_INS && i < 2 * S::DMA_INS) pp.copy_k(dk_r, j + 2, i - S::DMA_INS);
    if (NEXT && i >= NM1) {
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        // blocks in the order the QK^T steps finished them (kb descending)
        const int el = (i - NM1) * EPS + e, kb = S::NKB - 1 - (el >> 4), r = el & 15;
        if (MASK_NEXT)
          s_next[kb][r] = mask_score<CAUSAL>(s_next[kb][r], score_key(n1, kb, r, pp.g), pp.N, pp.qrow);
        mx = fmaxf(mx, s_next[kb][r]);
      }
      asm volatile("" : "+v"(mx));  // the running maximum advances step by step
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  st.l += lsum;
  if (NEXT) rescale<D>(st, max_halves(mx) * qk);  // after P_j V_j: acc and l hold tile j
}

// All iterations of one wave. nw: key tiles this wave visits, nfw: leading
// tiles it needs no mask for; the workgroup runs pp.n_tiles iterations, each
// ending with the copies' wait, the bf16 conversion and a barrier.
template <class S, bool IS_BF16, bool CONV_V, bool CAUSAL>
__device__ __forceinline__ void run_wave(const Pipe16<S> &pp, RowState16<S::D> &st, const u32x4 *qf,
                                         f32x16 (&sa)[S::NKB], f32x16 (&sb)[S::NKB], int nw, int nfw) {
  const int n = pp.n_tiles;
#define ITER(work)                                               \
  do {                                                           \
    work;                                                        \
    wait_vmcnt<0>(); /* K_{j+2} has landed */                   \
    lds_barrier();                                               \
  } while (0)
  int j = 0;
  const int n_a = max(min(nfw, nw) - 1, 0);  // tiles j < n_a have an unmasked successor
  for (; j + 2 <= n_a; j += 2) {
    ITER((iteration<S, IS_BF16, CONV_V, CAUSAL, false, true, 0>(pp, st, qf, j, sa, sb)));
    ITER((iteration<S, IS_BF16, CONV_V, CAUSAL, false, true, 1>(pp, st, qf, j + 1, sb, sa)));
  }
  if (j < n_a) {  // odd count of unmasked successors
    ITER((iteration<S, IS_BF16, CONV_V, CAUSAL, false, true, -1>(pp, st, qf, j, sa, sb)));
#pragma unroll
    for (int kb = 0; kb < S::NKB; ++kb) sa[kb] = sb[kb];
    ++j;
  }
  for (; j < nw - 1; ++j) {
    ITER((iteration<S, IS_BF16, CONV_V, CAUSAL, true, true, -1>(pp, st, qf, j, sa, sb)));
#pragma unroll
    for (int kb = 0; kb < S::NKB; ++kb) sa[kb] = sb[kb];
  }
  ITER((iteration<S, IS_BF16, CONV_V, CAUSAL, false, false, -1>(pp, st, qf, j, sa, sb)));
  // Tiles past this wave's rows: the same copies, conversion and waits.
  for (++j; j < n; ++j) {
    pp.issue_v(j + 1);
    pp.issue_k(j + 2);
    wait_vmcnt<S::DMA_INS>();
    pp.template convert_v<CONV_V>(j + 1);
    wait_vmcnt<0>();
    lds_barrier();
  }
#undef ITER
}

// bf16 V outside fp16's finite range. The P.V product runs on fp16 copies
// of bf16 V, so a value with |v| > 65504 became +-inf there and the
// accumulators of every wave that met it are not finite. Such a wave then
// recomputes its rows' outputs the way the page's kernel does, with P
// rounded to bf16 and V as the caller gave it (bf16 x bf16 on the matrix
// cores, fp32 accumulation), reading K and V straight from memory, against
// the final reference maximum: every score is within 2^kRescaleLog2 of it,
// so every weight stays <= 2^8. The rows' log-sum-exp is unchanged (it does
// not depend on V); the returned sum of the bf16-rounded weights normalises
// the new output. Inputs holding inf or NaN give non-finite outputs either
// way.
template <int D, bool CAUSAL, bool STRIDED>
__device__ __forceinline__ float redo_rows_bf16(const FwdParams &p, int bh, int r0, int qrow,
                                                int g, int l32, const u32x4 *qf,
                                                RowState16<D> &st) {
  constexpr int NKC = D / 16, NCB = D / 32;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const int N = STRIDED ? p.Nk : p.N;  // keys
  const size_t chead = (size_t)bh * (size_t)N * D;  // contiguous [B][H][N][D]
  const uint16_t *Kh = static_cast<const uint16_t *>(p.k) + (STRIDED ? head_off(p.ks, bh, p.H) : (int64_t)chead);
  const uint16_t *Vh =
      static_cast<const uint16_t *>(p.v_in) + (STRIDED ? head_off(p.vis, bh, p.H) : (int64_t)chead);
  const int64_t krs = STRIDED ? p.ks[2] : D, vrs = STRIDED ? p.vis[2] : D;
  const int dcol = STRIDED ? p.d : D;  // columns past dcol read as zeros
  const int kend = CAUSAL ? min(N, r0 + 32) : N;
  const float qk = p.qk, neg_m = st.neg_m;
  float l = 0.f;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) st.acc[cb] = f32x16{};
#pragma unroll 1
  for (int k0 = 0; k0 < kend; k0 += 32) {
    // S^T for keys k0 .. k0 + 31 (K operand row k0 + l32, as k_frag lays it out)
    const int key = k0 + l32;
    const uint16_t *krow = Kh + (int64_t)(key < N ? key : 0) * krs + 8 * g;
    f32x16 sc = f32x16{};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      u32x4 kf = u32x4{0, 0, 0, 0};
      if (STRIDED) {  // no load past column dcol: it may lie past the tensor
        if (key < N && 16 * kc + 8 * g < dcol) kf = *reinterpret_cast<const u32x4 *>(krow + 16 * kc);
      } else {
        kf = *reinterpret_cast<const u32x4 *>(krow + 16 * kc);
        if (key >= N) kf = u32x4{0, 0, 0, 0};
      }
      sc = mfma_qk<true>(kf, qf[kc], sc);
    }
    // weights, rounded to bf16 and packed as the P^T operands of the two
    // 16-key steps; the row sum takes the rounded values
    uint32_t pb[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      float w[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int kk = score_key(k0, 0, e + i, g);
        const bool dead = kk >= N || (CAUSAL && kk > qrow);
        w[i] = dead ? 0.f : exp2_fast(fmaf(sc[e + i], qk, neg_m));
      }
      const bf16x2 h = {(__bf16)w[0], (__bf16)w[1]};
      l += (float)h[0] + (float)h[1];
      pb[e >> 1] = __builtin_bit_cast(uint32_t, h);
    }
    // O^T += V^T P^T: the V^T operand of step (t, cb) is column 32cb + l32
    // at keys k0 + 16t + 8u + 4g + i (value 4u + i), loaded element by element
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pf = {pb[4 * t], pb[4 * t + 1], pb[4 * t + 2], pb[4 * t + 3]};
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        uint32_t vv[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int kk = k0 + 16 * t + 8 * (x >> 2) + 4 * g + (x & 3);
          vv[x] = kk < N && 32 * cb + l32 < dcol ? Vh[(int64_t)kk * vrs + 32 * cb + l32] : 0u;
        }
        const u32x4 a = {vv[0] | (vv[1] << 16), vv[2] | (vv[3] << 16), vv[4] | (vv[5] << 16),
                         vv[6] | (vv[7] << 16)};
        st.acc[cb] = mfma_qk<true>(a, pf, st.acc[cb]);
      }
    }
  }
  return l;
}

// Whether any accumulator of this lane is inf or NaN.
template <int D>
__device__ __forceinline__ bool acc_not_finite(const RowState16<D> &st) {
  bool bad = false;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) bad |= !__builtin_isfinite(st.acc[cb][r]);
  return bad;
}

// Row-major staging of one wave's 32 x D block of O in LDS for the
// epilogue: E bytes per element, rows of ROWB bytes (a whole row of O, or a
// MAXROWB-byte part of it when longer: PASSES parts), CPR 16-byte chunks per row,
// XOR-swizzled by row so the row-per-lane writes and the row-by-row reads
// spread over the banks; one wave instruction reads RPI rows.
template <int D, int E_, int MAXROWB>
struct OutStage {
  static constexpr int E = E_;
  static constexpr int ROWB = D * E > MAXROWB ? MAXROWB : D * E;
  static constexpr int PASSES = D * E / ROWB;
  static constexpr int CPR = ROWB / 16;
  static constexpr int RPI = 64 / CPR;
  static constexpr int COLS = ROWB / E;
  static constexpr int WAVE_BYTES = 32 * ROWB;
  __device__ static constexpr int swz(int row) { return row & (CPR - 1); }
};

// CONV_V: V arrives as bf16 and is converted in LDS; without it V is fp16
// already (fp16 inputs, or bf16 inputs whose V a first pass converted).
// One query tile (BLOCK_M rows of head bh) from the load of Q to the stores
// of O and LSE.
// prefetched: the previous tile of this workgroup (same head) already copied
// this tile's Q, V_0, K_0 and K_1. next_qt >= 0: copy that tile's ones once
// this tile's loop is done.
template <class S, bool IS_BF16, bool CAUSAL, bool OUT_F32, bool CONV_V, bool STRIDED>
__device__ __forceinline__ void attn_tile(const FwdParams &p, uint16_t *lds, int bh, int qt,
                                          bool prefetched, int next_qt) {
  constexpr int D = S::D;
  constexpr int BN = S::BN;
  constexpr int NCB = S::NCB;
  constexpr int NKC = S::NKC;

  // Opaque per call: the lane addresses derived from it are recomputed for
  // each tile instead of being held in registers across a workgroup's tiles.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  const int N = p.N;                       // query rows
  const int Nk = STRIDED ? p.Nk : N;       // keys
  const int m0 = qt * S::BLOCK_M;
  // Element offsets of this head and row strides: the tensors' own
  // (STRIDED), or those of contiguous [B][H][N][D] tensors, as constants.
  const size_t chead = (size_t)bh * (size_t)N * D;
  const uint16_t *Qh = static_cast<const uint16_t *>(p.q) + (STRIDED ? head_off(p.qs, bh, p.H) : (int64_t)chead);

  Pipe16<S> pp;
  pp.lds = lds;
  pp.Kh = static_cast<const uint16_t *>(p.k) + (STRIDED ? head_off(p.ks, bh, p.H) : (int64_t)chead);
  pp.Vh = static_cast<const uint16_t *>(p.v) + (STRIDED ? head_off(p.vs, bh, p.H) : (int64_t)chead);
  pp.qrs = STRIDED ? (int)p.qs[2] : D;
  pp.krs = STRIDED ? (int)p.ks[2] : D;
  pp.vrs = STRIDED ? (int)p.vs[2] : D;
  pp.dcol = STRIDED ? p.d : D;
  pp.la = lane_addr<D>(lane);
  pp.N = Nk;
  pp.Nq = N;
  pp.g = g;
  pp.tid = tid;
  pp.qk = p.qk;
  pp.lds_wave = __builtin_amdgcn_readfirstlane(lds_addr(lds) + wave * 1024);
  constexpr int RPI = S::THREADS / S::CPR;  // tile rows per copy instruction
#pragma unroll
  for (int c = 0; c < S::DMA_INS; ++c) {
    pp.k_dma[c] = dma_offset<D, false, STRIDED>(tid, pp.krs, pp.dcol) + (uint32_t)(c * RPI * pp.krs * 2);
    pp.v_dma[c] = dma_offset<D, true, STRIDED>(tid, pp.vrs, pp.dcol) + (uint32_t)(c * RPI * pp.vrs * 2);
  }
  pp.q_dma0 = dma_offset<D, false, STRIDED>(tid, pp.qrs, pp.dcol);
  // This lane's query row. Rows past N read zeros (the query tile's copy
  // descriptor is cut at N) and are never stored.
  const int r0 = m0 + wave * 32;  // first row of this wave
  pp.qrow = r0 + l32;


  // Key tiles to visit: for the workgroup (copies, barriers) and for this
  // wave (compute). Causal: only tiles holding some key <= the last row.
  // Tiles [0, nfw) need no mask for this wave.
  const int n_all = (Nk + BN - 1) / BN;
  const int n_tiles = CAUSAL ? min(n_all, (m0 + S::BLOCK_M + BN - 1) / BN) : n_all;
  const int nw = CAUSAL ? min(n_all, (r0 + 32 + BN - 1) / BN) : n_all;
  int nfw = Nk / BN;
  if (CAUSAL) nfw = min(nfw, (r0 + 1) / BN);
  pp.n_tiles = n_tiles;

  RowState16<D> st;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[cb][r] = 0.f;
  st.m = -INFINITY;
  st.neg_m = 0.f;
  st.l = 0.f;

  // Prologue: the query tile, V_0, K_0 and K_1 on their way (the query
  // tile through LDS: copied in whole rows, instead of 64 rows per load
  // instruction); V_0 (converted), Q and S_0 once Q, V_0 and K_0 are in;
  // K_1 in before iteration 0.
  if (prefetched) {
    wait_vmcnt<0>();  // also the previous tile's stores of O, issued later
  } else {
    pp.issue_q(Qh, m0);
    pp.issue_v(0);
    pp.issue_k(0);
    pp.issue_k(1);
    wait_vmcnt<S::DMA_INS>();  // Q, V_0, K_0
  }
  pp.template convert_v<CONV_V>(0);
  lds_barrier();
  u32x4 qf[NKC];  // Q[qrow][16kc + 8g .. +7], the B operand of QK^T
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) qf[kc] = k_frag<D>(pp.qstage(), pp.la, wave, kc);
  f32x16 sa[S::NKB], sb[S::NKB];  // scores of the current / next tile
  qk_tile<S, IS_BF16>(sa, qf, pp.kstage(0), pp.la);
  if (nfw == 0)
    softmax_max<S, CAUSAL, true>(st, sa, 0, Nk, pp.qrow, pp.qk, g);
  else
    softmax_max<S, CAUSAL, false>(st, sa, 0, Nk, pp.qrow, pp.qk, g);
  wait_vmcnt<0>();  // K_1
  lds_barrier();

  run_wave<S, IS_BF16, CONV_V, CAUSAL>(pp, st, qf, sa, sb, nw, nfw);

  // Copies issued for tiles past the end (empty byte ranges) retire before
  // the workgroup's LDS can be handed to another one.
  wait_vmcnt<0>();
  if (S::OWN_STAGE && next_qt >= 0) {
    // Every wave has passed the loop's last barrier: no one reads the ring
    // or the Q area any more. The next tile's first copies overlap this
    // tile's epilogue.
    const int m0n = next_qt * S::BLOCK_M;
    pp.n_tiles = CAUSAL ? min(n_all, (m0n + S::BLOCK_M + BN - 1) / BN) : n_all;
    pp.issue_q(Qh, m0n);
    pp.issue_v(0);
    pp.issue_k(0);
    pp.issue_k(1);
  }

  // Epilogue: combine the two key halves of the row sum, divide once, LSE.
  const float l_tot = sum_halves(st.l);
  const float l_safe = l_tot > 0.f ? l_tot : 1.f;
  float inv = 1.0f / l_safe;
  if (pp.qrow < N && g == 0)
    p.lse[(size_t)bh * N + pp.qrow] = (st.m + log2_fast(l_safe)) * 0.69314718055994531f;
  if (IS_BF16 && __any(acc_not_finite<D>(st))) {
    const float lb = sum_halves(redo_rows_bf16<D, CAUSAL, STRIDED>(p, bh, r0, pp.qrow, g, l32, qf, st));
    inv = 1.0f / (lb > 0.f ? lb : 1.f);
  }
  // O leaves through LDS. A lane holds one row, so stores straight from the
  // accumulators would touch 64 rows (64 cache lines) per instruction; staged
  // row-major, each store instruction writes whole lines. Each wave uses its
  // own slice of the staging area; when that is the ring, it is free once
  // every wave has passed this barrier (no copy is in flight).
  if (!S::OWN_STAGE) lds_barrier();
  using OS = OutStage<D, OUT_F32 ? 4 : 2, S::STAGE_ROWB>;
  static_assert(S::WAVES * OS::WAVE_BYTES <= (S::OWN_STAGE ? S::STAGE_ELEMS * 2 : S::RING_ELEMS * 2),
                "staging fits");
  uint8_t *stage = reinterpret_cast<uint8_t *>(lds + (S::OWN_STAGE ? S::RING_ELEMS + S::BLOCK_M * D : 0)) +
                   wave * OS::WAVE_BYTES;
  const int64_t ors = STRIDED ? p.os[2] : D;
  uint8_t *obase = static_cast<uint8_t *>(p.o) +
                   ((STRIDED ? head_off(p.os, bh, p.H) : (int64_t)chead) + (int64_t)r0 * ors) * OS::E;
#pragma unroll
  for (int ps = 0; ps < OS::PASSES; ++ps) {
    // This lane's row l32: 4-column pieces at 32cb + 8r4 + 4g.
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = cb * 32 + r4 * 8 + g * 4 - ps * OS::COLS;
        if (col < 0 || col >= OS::COLS) continue;
        const int byte = col * OS::E;
        uint8_t *dst = stage + l32 * OS::ROWB + (((byte >> 4) ^ OS::swz(l32)) << 4) + (byte & 15);
        const float o0 = st.acc[cb][4 * r4 + 0] * inv, o1 = st.acc[cb][4 * r4 + 1] * inv;
        const float o2 = st.acc[cb][4 * r4 + 2] * inv, o3 = st.acc[cb][4 * r4 + 3] * inv;
        if (OUT_F32) {
          *reinterpret_cast<f32x4 *>(dst) = f32x4{o0, o1, o2, o3};
        } else if (IS_BF16) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          *reinterpret_cast<bf16x4 *>(dst) = bf16x4{(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3};
        } else {
          typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
          *reinterpret_cast<f16x4 *>(dst) =
              f16x4{(_Float16)o0, (_Float16)o1, (_Float16)o2, (_Float16)o3};
        }
      }
    __builtin_amdgcn_wave_barrier();
    // Read back by rows: lane = (row within the group, 16-byte chunk).
#pragma unroll
    for (int k = 0; k < 32 / OS::RPI; ++k) {
      const int row = k * OS::RPI + lane / OS::CPR, c = lane % OS::CPR;
      const u32x4 val =
          *reinterpret_cast<const u32x4 *>(stage + row * OS::ROWB + ((c ^ OS::swz(row)) << 4));
      // strided instances: 16-byte pieces at or past column d are not stored
      if (r0 + row < N && (!STRIDED || (ps * OS::ROWB + c * 16) / OS::E < pp.dcol))
      {
        u32x4 *dst = reinterpret_cast<u32x4 *>(obase + (int64_t)row * ors * OS::E + ps * OS::ROWB + c * 16);
        if (ATTN_CFG_O_NONTEMPORAL) __builtin_nontemporal_store(val, dst); else *dst = val;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Causal query tiles differ in length (tile t visits about t+1 key tiles),
// and with one tile per workgroup the last workgroups to finish leave CUs
// idle. A causal workgroup therefore takes tile nq-1-i and then tile i: all
// pairs are equally long (the middle tile of an odd count runs alone, last).
// Workgroups are handed to the 8 XCDs round-robin (id w runs on XCD w % 8)
// and start in id order within an XCD. When B*H is a multiple of 8, the ids
// of one XCD run head-major: all work items of head bh sit on XCD bh % 8 and
// start together, so each head's K/V stream through that XCD's L2 about once
// rather than once per wave of workgroups. Otherwise ids run item-major,
// head-minor.
template <class S, bool IS_BF16, bool CAUSAL, bool OUT_F32, bool CONV_V, bool STRIDED>
__global__ __launch_bounds__(S::THREADS, S::WG_PER_CU) void attn_fwd_16(FwdParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::LDS_ELEMS];
  const int w = blockIdx.x;
  int t, bh;
  if ((p.BH & 7) == 0) {
    const int per_head = CAUSAL && ATTN_CFG_CAUSAL_PAIRS ? (p.nq + 1) >> 1 : p.nq;
    const int j = w >> 3;
    const int hl = j / per_head;
    t = j - hl * per_head;
    bh = ATTN_CFG_HEAD_BLOCKED ? (w & 7) * (p.BH >> 3) + hl : (hl << 3) | (w & 7);
  } else {
    t = w / p.BH;
    bh = w - t * p.BH;
  }
  if (CAUSAL && !ATTN_CFG_CAUSAL_PAIRS) {
    attn_tile<S, IS_BF16, CAUSAL, OUT_F32, CONV_V, STRIDED>(p, lds, bh, p.nq - 1 - t, false, -1);
    return;
  }
  if (!CAUSAL) {
    attn_tile<S, IS_BF16, CAUSAL, OUT_F32, CONV_V, STRIDED>(p, lds, bh, t, false, -1);
    return;
  }
  const int q_long = p.nq - 1 - t, q_short = t;
  const int n_items = q_short < q_long ? 2 : 1;
  const bool short_first = n_items == 2 && (ATTN_CFG_CAUSAL_SHORT_FIRST == 1 ||
                                             (ATTN_CFG_CAUSAL_SHORT_FIRST == 2 && (t & 1)));
  const int qa = short_first ? q_short : q_long;
  const int qb = short_first ? q_long : q_short;
#pragma unroll 1
  for (int k = 0; k < n_items; ++k) {
    // The second tile's copies reuse the LDS the first one's epilogue read.
    if (k > 0) lds_barrier();
    attn_tile<S, IS_BF16, CAUSAL, OUT_F32, CONV_V, STRIDED>(p, lds, bh, k == 0 ? qa : qb,
                                                   S::OWN_STAGE && k > 0,
                                                   k + 1 < n_items ? qb : -1);
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
// First pass for long bf16 sequences: V -> fp16 into a workspace, once per
// element, instead of once per query tile inside the attention kernel (the
// same rounding: exact for |v| in [2^-14, 65504]). Eight values per thread
// per step of a grid-stride loop; n8 counts groups of eight.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void v_to_f16(const u32x4 *src, u32x4 *dst, int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const u32x4 x = src[i];
    u32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = pack_f16(bf16_lo_to_f32(x[e]), bf16_hi_to_f32(x[e]));
    dst[i] = y;
  }
}
constexpr int kPrepassBlocks = 8192;
// The first pass costs about as much as the in-LDS conversion saves at
// N = 4096 (causal) and pays off from about twice that: kernel time grows
// with N^2, the pass with N.
constexpr int64_t kPrepassMinN = ATTN_CFG_PREPASS_MIN_N;
// Largest row stride (elements) of a strided tensor the tuned kernels take:
// a query tile of up to 256 rows then spans less than 2^31 bytes, the range
// of a buffer descriptor and of the 32-bit copy offsets.
constexpr int64_t kMaxRowStride = int64_t(1) << 21;

// --------------------------------------------------------------------------
// Host side: validation, dispatch, launch.
// --------------------------------------------------------------------------
typedef void (*KernelFn)(FwdParams);

// A bf16/fp16 kernel and its launch shape.
struct Launch16 {
  KernelFn fn;
  int block_m;       // query rows per workgroup
  unsigned threads;  // threads per workgroup
};

// Strided tensors: a kernel instance of its own, so the contiguous one keeps
// its strides as compile-time constants; no first pass (bf16 V is converted
// in LDS).
template <class S, bool IS_BF16, bool CAUSAL>
KernelFn pick16(bool out_f32, bool conv_v, bool strided) {
  if (strided)
    return out_f32 ? attn_fwd_16<S, IS_BF16, CAUSAL, true, IS_BF16, true>
                   : attn_fwd_16<S, IS_BF16, CAUSAL, false, IS_BF16, true>;
  if (IS_BF16 && conv_v)
    return out_f32 ? attn_fwd_16<S, IS_BF16, CAUSAL, true, IS_BF16, false>
                   : attn_fwd_16<S, IS_BF16, CAUSAL, false, IS_BF16, false>;
  return out_f32 ? attn_fwd_16<S, IS_BF16, CAUSAL, true, false, false>
                 : attn_fwd_16<S, IS_BF16, CAUSAL, false, false, false>;
}

template <class S>
Launch16 launch16(attn_dtype in, bool out_f32, bool causal, bool conv_v, bool strided) {
  KernelFn fn;
  if (in == ATTN_BF16)
    fn = causal ? pick16<S, true, true>(out_f32, conv_v, strided)
                : pick16<S, true, false>(out_f32, conv_v, strided);
  else
    fn = causal ? pick16<S, false, true>(out_f32, false, strided)
                : pick16<S, false, false>(out_f32, false, strided);
  return Launch16{fn, S::BLOCK_M, (unsigned)S::THREADS};
}

// The tile of a problem. The pages key their autotuning on the sequence
// length, the head dimension and the mask; here two compiled tiles per head
// dimension compete: 8 waves (one 256-row workgroup per CU; d=128: 64-key
// tiles, d=64: 128-key) and 4 waves (128-row workgroups; d=128: 32-key
// tiles, two per CU; d=64: 64-key tiles, whose 48 KB of LDS and at most 168
// VGPRs let three share a CU). Measured at full occupancy, the 8-wave tile
// is faster per unit of work (5% at d=64, 10% at d=128), but the grid runs
// in whole rounds of workgroups: a last round that is only partly filled
// leaves CUs idle for a whole workgroup's time, and with 4-wave tiles a
// last round of at most one workgroup per CU runs each alone on its CU,
// faster (taken as 0.6 of a round). Each tile's cost is its number of
// rounds so weighted, times its per-unit cost; the cheaper one is taken.
// The rounds are counted at two 4-wave workgroups per CU for both head
// dimensions: the constants were fitted to measurements
// (io_aware_attention_flash_amd/sweep.py timed every tile on workloads with
// whole and partial last rounds; this rule picks the fastest tile, or one
// within 0.3% of it, on each), and counting three at d=64 with the same
// constants would pick the 4-wave tile at B4 H16 N2048, where it is 2%
// slower.
constexpr int kCUs = 256;

double tile_cost(int64_t units, int wg_per_cu, double unit_cost) {
  const double rounds = (double)units / (double)(kCUs * wg_per_cu);
  const double full = (double)(int64_t)rounds, frac = rounds - full;
  double last = 0.0;
  if (frac > 0.0) last = wg_per_cu == 2 && frac <= 0.5 ? 0.6 : 1.0;
  return (full + last) * unit_cost;
}

// Whether the 8-wave tile is the cheaper one for B*H heads of N rows.
bool pick_wide(int64_t BH, int64_t N, bool causal, double narrow_unit_cost) {
  const int64_t nq8 = (N + 255) / 256, nq4 = (N + 127) / 128;
  const int64_t u8 = (causal ? (nq8 + 1) / 2 : nq8) * BH;
  const int64_t u4 = (causal ? (nq4 + 1) / 2 : nq4) * BH;
  return tile_cost(u8, 1, 1.0) <= tile_cost(u4, 2, narrow_unit_cost);
}

Launch16 pick_launch16(int64_t d, int64_t BH, int64_t N, int64_t Nk, attn_dtype in, bool out_f32,
                       bool causal, bool conv_v, bool strided) {
  if (d == 128) {
#if ATTN_FWD_D128_FORCED
    (void)BH;
    return launch16<Tile16<128>>(in, out_f32, causal, conv_v, strided);
#else
    if (pick_wide(BH, N, causal, 1.10))
      return launch16<Shape16<128, 8, 64>>(in, out_f32, causal, conv_v, strided);
    return launch16<Shape16<128, 4, 32>>(in, out_f32, causal, conv_v, strided);
#endif
  }
#if ATTN_FWD_D64_FORCED
  (void)Nk;
  return launch16<Tile16<64>>(in, out_f32, causal, conv_v, strided);
#else
  // With fewer than 256 keys most of the 8-wave tile's 128-key stages would
  // be masked: the 64-key tile (measured 17-27% faster at 77-255 keys).
  if (Nk >= 256 && pick_wide(BH, N, causal, 1.05))
    return launch16<Shape16<64, 8, 128>>(in, out_f32, causal, conv_v, strided);
  return launch16<Shape16<64, 4, 64>>(in, out_f32, causal, conv_v, strided);
#endif
}

// Bytes of the fp16 copy of V the first pass writes, or 0 when the problem
// does not take the first pass (or is invalid).
size_t prepass_bytes(int64_t B, int64_t H, int64_t N, int64_t d, attn_dtype in_dtype) {
  if (in_dtype != ATTN_BF16 || N < kPrepassMinN || (d != 64 && d != 128)) return 0;
  if (B < 1 || H < 1 || N > (int64_t(1) << 24) || B * H > (int64_t(1) << 24)) return 0;
  return (size_t)(B * H) * (size_t)N * (size_t)d * 2;
}

thread_local int g_last_hip_error = 0;

}  // namespace

// The backward's translation unit reports launch errors through the same
// per-thread slot that attn_last_hip_error() reads.
extern "C" {
static attn_status attn_fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse,
                                 int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                 float scale, attn_dtype in_dtype, attn_dtype out_dtype,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 const int64_t *strides, int64_t Nk);
}

namespace attn_internal {
void set_last_hip_error(int e) { g_last_hip_error = e; }

// Whether the tuned bf16/fp16 kernels take a strided problem of
// attn_fwd_strided (self- or cross-attention; the caller has checked that a
// causal problem has equal query and key lengths, and that d is a multiple
// of 8 up to 128): bf16/fp16 inputs, and row strides whose tiles fit a
// buffer descriptor's 32-bit range. st holds the (batch, head, row) strides
// of q, k, v and o, validated by the caller.
bool fwd16_takes_strided(int64_t Nk, int64_t d, attn_dtype in_dtype, const int64_t *st) {
  (void)Nk, (void)d;
  if (in_dtype != ATTN_BF16 && in_dtype != ATTN_F16) return false;
  for (int t = 0; t < 4; ++t)
    if (st[3 * t + 2] < d || st[3 * t + 2] > kMaxRowStride) return false;
  return true;
}

attn_status fwd16_strided(const void *q, const void *k, const void *v, void *o, float *lse,
                          int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                          float scale, attn_dtype in_dtype, attn_dtype out_dtype, void *stream,
                          const int64_t *st) {
  return attn_fwd_impl(q, k, v, o, lse, B, H, Nq, d, causal, scale, in_dtype, out_dtype, nullptr, 0,
                       stream, st, Nk);
}
}  // namespace attn_internal

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
    case ATTN_ERR_WORKSPACE: return "workspace missing, too small or not 16-byte aligned";
    case ATTN_ERR_CAPACITY: return "problem larger than the static scratch of the allocation-free entry point";
  }
  return "unknown status";
}

// strides: NULL for contiguous [B][H][N][d] tensors, else the (batch, head,
// row) element strides of q, k, v and o, 12 values, already validated
// (bf16/fp16 inputs, rows 16-byte aligned, row strides in [d, kMaxRowStride]).
// Nk: keys per head; it may differ from N (query rows) only with strides and
// without the causal mask.
static attn_status attn_fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse,
                                 int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                 float scale, attn_dtype in_dtype, attn_dtype out_dtype,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 const int64_t *strides, int64_t Nk) {
  // Validation first: no HIP call happens before every argument is checked.
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1 || Nk < 1) return ATTN_ERR_SHAPE;
  if (N > (int64_t(1) << 24) || Nk > (int64_t(1) << 24) || B * H > (int64_t(1) << 24))
    return ATTN_ERR_SHAPE;
  if (Nk != N && (!strides || causal)) return ATTN_ERR_SHAPE;
  // Contiguous tensors: d = 64 or 128. Strided ones: a multiple of 8 up to
  // 128, computed at D = 64 or 128 with zero columns.
  if (strides ? (d < 8 || d > 128 || d % 8 != 0) : (d != 64 && d != 128))
    return ATTN_ERR_UNSUPPORTED;
  const int64_t D = d <= 64 ? 64 : 128;
  if (strides && in_dtype != ATTN_BF16 && in_dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
  const bool in_ok = in_dtype == ATTN_F32 || in_dtype == ATTN_F16 || in_dtype == ATTN_BF16;
  if (!in_ok) return ATTN_ERR_UNSUPPORTED;
  if (in_dtype == ATTN_F32 && out_dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (in_dtype != ATTN_F32 && out_dtype != in_dtype && out_dtype != ATTN_F32)
    return ATTN_ERR_UNSUPPORTED;
  if (!(scale >= 0.f) || !isfinite(scale)) return ATTN_ERR_SCALE;
  // The first pass runs when the problem takes it and the workspace can hold
  // its output (16-byte aligned); otherwise the kernel converts V in LDS.
  // Both give the same bits.
  const size_t need = strides ? 0 : prepass_bytes(B, H, N, d, in_dtype);
  const bool prepass = need > 0 && workspace != nullptr && workspace_bytes >= need &&
                       (reinterpret_cast<uintptr_t>(workspace) & 15) == 0;
  const bool out_f32 = out_dtype == ATTN_F32;
  // The kernel, and its query rows and threads per workgroup.
  const bool f32_path = in_dtype == ATTN_F32;
  Launch16 l16 = {nullptr, 0, 0};
  if (!f32_path)
    l16 = pick_launch16(D, B * H, N, Nk, in_dtype, out_f32, causal != 0, !prepass, strides != nullptr);
  const int64_t block_m = f32_path ? kBlockM : l16.block_m;
  const unsigned threads = f32_path ? kThreads : l16.threads;
  const int64_t nq = (N + block_m - 1) / block_m;
  // Causal bf16/fp16 workgroups take two query tiles each (long + short).
  const int64_t grid = (causal && !f32_path && ATTN_CFG_CAUSAL_PAIRS ? (nq + 1) / 2 : nq) * B * H;
  if (grid > INT32_MAX) return ATTN_ERR_SHAPE;

  FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.v_in = v;
  p.o = o;
  p.lse = lse;
  const int64_t cont[3] = {H * N * d, N * d, d};
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = strides ? strides[i] : cont[i];
    p.ks[i] = strides ? strides[3 + i] : cont[i];
    p.vs[i] = p.vis[i] = strides ? strides[6 + i] : cont[i];
    p.os[i] = strides ? strides[9 + i] : cont[i];
  }
  p.d = (int)d;
  p.N = (int)N;
  p.Nk = (int)Nk;
  p.nq = (int)nq;
  p.BH = (int)(B * H);
  p.H = (int)H;
  // scale * log2(e) in double, rounded once; a zero scale becomes FLT_MIN so
  // masked scores (-inf) never meet a 0 factor.
  double qk = (double)scale * 1.4426950408889634;
  p.qk = qk < (double)FLT_MIN ? FLT_MIN : (float)qk;

  KernelFn fn = l16.fn;
  if (f32_path)
    fn = d == 64 ? (causal ? attn_fwd_f32<64, true> : attn_fwd_f32<64, false>)
                 : (causal ? attn_fwd_f32<128, true> : attn_fwd_f32<128, false>);
  hipStream_t st = (hipStream_t)stream;
  hipError_t err = hipSuccess;
  if (prepass) {
    int64_t n8 = (int64_t)(need / 16);
    const int64_t blocks = (n8 + 255) / 256 < kPrepassBlocks ? (n8 + 255) / 256 : kPrepassBlocks;
    const void *src = v;
    void *cargs[] = {&src, &workspace, &n8};
    err = hipLaunchKernel(reinterpret_cast<const void *>(v_to_f16), dim3((unsigned)blocks),
                          dim3(256), cargs, 0, st);
    p.v = workspace;  // contiguous, like the caller's V (p.vis)
  }
  if (err == hipSuccess) {
    void *args[] = {&p};
    err = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((unsigned)grid), dim3(threads),
                          args, 0, st);
  }
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                     int64_t H, int64_t N, int64_t d, int causal, float scale, attn_dtype in_dtype,
                     attn_dtype out_dtype, void *stream) {
  return attn_fwd_impl(q, k, v, o, lse, B, H, N, d, causal, scale, in_dtype, out_dtype, nullptr, 0,
                       stream, nullptr, N);
}

size_t attn_fwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, attn_dtype in_dtype) {
  return prepass_bytes(B, H, N, d, in_dtype);
}

attn_status attn_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                        attn_dtype in_dtype, attn_dtype out_dtype, void *workspace,
                        size_t workspace_bytes, void *stream) {
  return attn_fwd_impl(q, k, v, o, lse, B, H, N, d, causal, scale, in_dtype, out_dtype, workspace,
                       workspace_bytes, stream, nullptr, N);
}

}  // extern "C"
