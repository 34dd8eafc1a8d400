// Blockwise causal attention with the online-softmax update, bf16 MFMA on gfx950.
//
// What is computed ([Digest] = "从 Ring Attention 到 DeepSpeed Ulysses，再到 USP 统一框架",
// jsqmd.com): softmax(Q K^T / sqrt(d)) V (§2) of one Q share against the KV shares of a
// range of ring steps (§3.1, §3.3), each KV tile folded into the running (m, l, O) of every
// query row by the update of §3.2, whose result does not depend on the order the tiles are
// folded in (up to rounding). Masked pairs follow the causal matrix of §3.4 by global
// position.
//
// Mapping onto CDNA4:
//  * A workgroup of 4 wave64s owns BM query rows of one (batch, head); each wave owns QB blocks
//    of 32 rows and lane l owns query row (l mod 32) of each block. Every K or V operand read
//    from LDS feeds one MFMA per block.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K tile rows
//    from LDS are the A operand, the wave's Q rows (held in VGPRs for the whole kernel) are
//    the B operand. The 32x32 fp32 result leaves each lane with 16 keys of its own query, so
//    the row max and row sum are in-lane reductions plus one v_permlane32_swap.
//  * O^T += V^T P^T with the same instruction: P^T is the score accumulator converted to
//    bf16 in place (no data movement). V stays in LDS in its natural [key][d] layout and the
//    transposed A operand is read with ds_read_b64_tr_b16, which hands each lane one head-dim
//    column of a 4-key x 16-column block; two such reads give the 8 keys that match, key for
//    key, the order in which the score accumulator feeds the B operand.
//  * K/V tiles (64 keys) go from HBM straight into LDS with buffer_load_dwordx4 ... lds (each
//    lane moves 16 bytes, a wave 1 KB), so staging costs no registers and no LDS-write
//    instructions; the buffer resource covers only the tile's valid rows, so the rows of a
//    ragged last tile arrive as zeros. Rows are unpadded; the 16-byte chunks of each row are XOR-permuted by a
//    function of the key so that the 128-bit K reads and the transposed V reads hit distinct
//    banks. The staging is staggered so that, while tile j is in the softmax, K of tile j+1
//    and V of tile j are resident: the next tile's QK^T MFMAs are issued in the same block as
//    this tile's softmax VALU work and the two overlap. One barrier per tile.
//  * Tiles whose keys are all invisible to the workgroup's rows are never visited: the
//    visible keys of a share form a prefix (positions increase along a share), whose length
//    comes from the position rule. Only tiles straddling the causal boundary or the ragged
//    tail evaluate the mask. Workgroups are launched heaviest query tile first.
//  * Short shares (fewer query tiles than two per CU) run a workgroup of two such wave groups
//    on the same query rows, each folding every other key tile of the sequence into its own
//    (m, l, O); the two states are merged through LDS at the end with the log-sum-exp update.
//    That puts two waves on every SIMD where one workgroup per query tile would leave one.
//  * Striped shares on large grids pair query tiles n_qt-1-p and p in one workgroup, the second
//    walked backward over its key tiles: every workgroup then has the same work, and the
//    resident ones read the same key tiles at the same time (shared in L2).
//  * The body of one query tile is in attn_bf16_tile.inc, expanded in place for one tile per
//    workgroup and inside a lambda (once per direction) for a pair.
//  * The softmax runs in the log2 domain (exp2 of scores pre-multiplied by scale*log2 e), with
//    the exact running max as reference, so the largest weight so far is exactly 1 in bf16 (this
//    keeps peaked softmaxes accurate). O and l are rescaled only on tiles where some row's max
//    grows (a wave-uniform branch, rarely taken once the first tiles have been seen). LSE is
//    converted back to the natural log at the end.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <type_traits>
#include <utility>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int QB = RA_ATTN_QB;    // 32-row query blocks per wave
constexpr int WR = 32 * QB;       // query rows per wave
constexpr int BM = kBf16BlockM;   // query rows per workgroup
constexpr int BN = kBf16BlockN;   // keys per tile
constexpr int NT = 64 * RA_ATTN_WAVES;  // threads per workgroup
static_assert(BM == WR * RA_ATTN_WAVES, "block shape");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

#ifndef RA_ATTN_SCHED
#define RA_ATTN_SCHED 1               // pin the MFMA / VALU / LDS-read interleave of the main block
#endif
#ifndef RA_ATTN_SCHED_VALU
#define RA_ATTN_SCHED_VALU 3          // VALU ops placed after each MFMA of the main block
#endif
#ifndef RA_ATTN_SCHED_AHEAD
#define RA_ATTN_SCHED_AHEAD 6         // LDS operand reads issued before the first MFMA
#endif
#ifndef RA_ATTN_SETPRIO
#define RA_ATTN_SETPRIO 1             // raise wave priority while issuing the main block
#endif
#ifndef RA_ATTN_TILE_GROUP
#define RA_ATTN_TILE_GROUP 32         // consecutive tiles of one step visited before the next step
#endif
#ifndef RA_ATTN_MUL24
#define RA_ATTN_MUL24 1               // 24-bit multiply for the copies' row offsets (rows < 2^24 bytes)
#endif
#ifndef RA_ATTN_SCHED_FIRST
#define RA_ATTN_SCHED_FIRST 44        // VALU ops placed before the first MFMA of the main block
#endif
#ifndef RA_ATTN_KVS_GROUP_SYNC
#define RA_ATTN_KVS_GROUP_SYNC 1      // key split: each wave group synchronises only its own waves per tile
#endif
#ifndef RA_ATTN_SOFFSET
#define RA_ATTN_SOFFSET 1             // the copies' wave-uniform row offset as the scalar offset
#endif
#ifndef RA_ATTN_DMA_REGS
#define RA_ATTN_DMA_REGS 0            // keep the lanes' copy offsets in registers for the whole loop
#endif
#ifndef RA_ATTN_TILE_GROUP_PAIR
#define RA_ATTN_TILE_GROUP_PAIR RA_ATTN_TILE_GROUP  // the same for paired query tiles of long shares
#endif
#ifndef RA_ATTN_TILE_GROUP_SHORT
#define RA_ATTN_TILE_GROUP_SHORT 8    // paired query tiles of short shares (PAIR = 2)
#endif
#ifndef RA_ATTN_SHORT_SHARE
#define RA_ATTN_SHORT_SHARE 8192      // K/V shares of at most this many rows count as short
#endif
#ifndef RA_ATTN_WAVES_PER_SIMD
#define RA_ATTN_WAVES_PER_SIMD 2      // occupancy target: 256 VGPRs per wave at 2, 512 at 1
#endif

constexpr int TG_ONE = RA_ATTN_TILE_GROUP;
constexpr int TG_PAIR = RA_ATTN_TILE_GROUP_PAIR;
constexpr int TG_SHORT = RA_ATTN_TILE_GROUP_SHORT;

// Word 3 of a raw buffer resource (untyped 32-bit data, no swizzle, no stride): reads past
// num_records return zeros.
constexpr int kBufferWord3 = 0x00020000;

template <int D>
struct Cfg {
  static constexpr int ROWB = D * 2;               // bytes per K/V row in LDS (unpadded)
  static constexpr int SPR = D / 8;                // 16-byte chunks per row
  static constexpr int RPB = 256 / ROWB;           // rows per 256-byte sweep of the banks
  static constexpr int ELEMS = BN * D;             // one tile of K or V
  static constexpr int NWAVE = NT / 64;
  static constexpr int DMA = BN * ROWB / 1024 / NWAVE;  // 1 KB global->LDS copies per wave
  static_assert(BN * ROWB % (1024 * NWAVE) == 0, "tile copy must divide evenly over the waves");
  static_assert(SPR >= 8, "swizzles assume at least 8 chunks per row");
  // Physical chunk of logical chunk c of row `key`. K: 16 lanes read one logical chunk of 16
  // consecutive keys. V: a transposed read covers 4 consecutive keys x 4 consecutive chunks.
  static __host__ __device__ constexpr int k_swz(int key) { return (key / RPB) & (SPR - 1); }
  static __host__ __device__ constexpr int v_swz(int key) { return (4 * ((key / RPB) & 3)) & (SPR - 1); }
};

struct OutBf16 {
  static __device__ inline void store4(void* base, int64_t off, f32x4 x) {
    bf16x4 y;
    y[0] = (__bf16)x[0];
    y[1] = (__bf16)x[1];
    y[2] = (__bf16)x[2];
    y[3] = (__bf16)x[3];
    *(bf16x4*)((__bf16*)base + off) = y;
  }
};
struct OutF32 {
  static __device__ inline void store4(void* base, int64_t off, f32x4 x) {
    *(f32x4*)((float*)base + off) = x;
  }
};

// Partner lane l^32 combined with the own value: v_permlane32_swap hands every lane both its
// own value and its partner's (in one order or the other), so max/sum of the pair is exact.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline s16x4 read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Position in the (step, tile) sequence a workgroup walks: tile t of the share of ring step s,
// whose first nf tiles are fully visible to the workgroup; the step's K/V rank and its share
// pointers at the workgroup's batch and head.
struct Cursor {
  int s, t, nt, nf, rank;
  const char* kb;
  const char* vb;
};

// Scheduling groups of one chunk of the main block: NM MFMAs, each followed by an even share
// of the chunk's NV VALU ops and ND LDS reads.
template <int Mask, int N>
__device__ __forceinline__ void sched_group() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(Mask, N, 0);
}
template <int NM, int NV, int ND, int... I>
__device__ __forceinline__ void sched_chunk(std::integer_sequence<int, I...>) {
  ((sched_group<0x008, 1>(), sched_group<0x002, (I + 1) * NV / NM - I * NV / NM>(),
    sched_group<0x100, (I + 1) * ND / NM - I * ND / NM>()),
   ...);
}

// KVS = 1: one group of RA_ATTN_WAVES waves visits every K/V tile of the workgroup's sequence.
// KVS = 2 (grids too small to put two workgroups on every CU): two such groups own the same
// query rows, group g folding the tiles at odd (g = 1) or even (g = 0) places of the sequence
// into its own (m, l, O); the groups' states are merged through LDS at the end, like two
// blocks of the ring merged by the log-sum-exp update. Each SIMD then holds two waves.
// PAIR = 1 or 2 (striped shares on large grids): a workgroup takes the query tiles n_qt-1-p and p.
// Under a causal mask a query tile's work grows linearly with its index, so every pair has the
// same total; the first tile walks its (step, tile) sequence forward and the second backward,
// so the workgroups resident at once read the same key tiles at the same time and finish
// together (unpaired, the striped share's late-starting workgroups walk out of step with the
// running ones and miss in L2).
// DBG = 1 (debug hook only, never a product launch): every wave also counts the K/V tiles it
// folds in, those on which it evaluates the mask, and two kinds of fault that a correct walk
// never shows (a copied or folded tile outside its step's visible tiles, a folded tile that no
// query row of the tile sees), and writes the four counts to a.dbg_counts.
template <int D, class Out, int KVS, int PAIR, int DBG>
__global__ __launch_bounds__(NT * KVS, QB == 1 ? RA_ATTN_WAVES_PER_SIMD : 1) void attn_bf16_kernel(const AttnArgs a) {
  using C = Cfg<D>;
  static_assert(KVS == 1 || (KVS == 2 && QB == 1), "the key split merges one 32-row block per wave");
  static_assert(PAIR == 0 || KVS == 1, "pairing and the key split are not combined");
  // The two stages of K and V are four distinct LDS objects: the copies into one stage and the
  // reads of the other can then be told apart, so no wait for in-flight copies is inserted
  // before the reads.
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds0[C::ELEMS * KVS];
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds1[C::ELEMS * KVS];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds0[C::ELEMS * KVS];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds1[C::ELEMS * KVS];
  // Key split: arrival counters of the two wave groups' own barrier (each group stages its tiles
  // in its own LDS regions, so within the tile loop a group only waits for its own waves).
  __shared__ uint32_t grp_sync[2];

  // tiles of one step visited before the next step
  constexpr int TG = PAIR == 2 ? TG_SHORT : (PAIR ? TG_PAIR : TG_ONE);
  const int tid = threadIdx.x;
  const int wave_wg = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep in SGPRs
  const int grp = KVS == 1 ? 0 : wave_wg / RA_ATTN_WAVES;        // key-split group
  const int wave = KVS == 1 ? wave_wg : wave_wg % RA_ATTN_WAVES;  // wave within the group
  const int goff = grp * C::ELEMS;                                // the group's LDS tiles
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  if (KVS == 2 && tid < 2) grp_sync[tid] = 0;  // visible to all waves after the prologue's barriers

  const int nbh = a.B * a.H;
  const int n_qt = (a.Sq + BM - 1) / BM;
  const int bh = blockIdx.x % nbh;
  const int pidx = (int)(blockIdx.x / nbh);
  const int qt_first = n_qt - 1 - pidx;  // heaviest (latest) query tile first
  const int b = bh / a.H;
  // Consecutive workgroups go to the 8 XCDs in turn, so head (bh mod H) runs on XCD
  // (bh mod 8) when 8 divides H. With grouped KV heads the heads are renumbered so that each
  // XCD takes a contiguous run of H/8 heads: the query heads sharing a KV head then share one
  // XCD's L2 instead of each XCD reading every KV head.
  const int hr = bh % a.H;
  const int h = (a.Hkv < a.H && a.H % 8 == 0) ? (hr % 8) * (a.H / 8) + hr / 8 : hr;
  // The body of one query tile (attn_bf16_tile.inc) is expanded in place for one tile per
  // workgroup, and inside a lambda called once per direction for a pair of tiles, so that the
  // one-tile kernel compiles exactly as a plain kernel body would.
  if constexpr (PAIR == 0) {
    const int qt = qt_first;
    constexpr bool kRev = false;
#include "attn_bf16_tile.inc"
  } else {
    auto run_tile = [&](auto rev_c, const int qt) {
      constexpr bool kRev = decltype(rev_c)::value;
#include "attn_bf16_tile.inc"
    };
    run_tile(std::false_type(), qt_first);
    if (pidx < n_qt - 1 - pidx) {
      __syncthreads();  // every wave is done with the first tile's LDS stages
      run_tile(std::true_type(), pidx);
    }
  }
}

}  // namespace

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// RA_KV_SPLIT override of the automatic key-split choice: 1 "always", -1 "never", 0 automatic.
static int kv_split_override() {
  const char* e = getenv("RA_KV_SPLIT");
  if (!e) return 0;
  if (!strcmp(e, "always")) return 1;
  if (!strcmp(e, "never")) return -1;
  return 0;
}

// RA_PAIR_TILES override of the automatic pairing choice: 1 "always", -1 "never", 0 automatic.
static int pair_override() {
  const char* e = getenv("RA_PAIR_TILES");
  if (!e) return 0;
  if (!strcmp(e, "always")) return 1;
  if (!strcmp(e, "never")) return -1;
  return 0;
}

// RA_PAIR_GROUP override of the paired kernels' tile-group size: 1 "long" (groups of 32 tiles),
// -1 "short" (groups of 8), 0 automatic (short for K/V shares of at most RA_ATTN_SHORT_SHARE rows).
static int pair_group_override() {
  const char* e = getenv("RA_PAIR_GROUP");
  if (!e) return 0;
  if (!strcmp(e, "long")) return 1;
  if (!strcmp(e, "short")) return -1;
  return 0;
}

template <int KVS, int PAIR, int DBG>
static void launch_dbg(const AttnArgs& a, int D, int o_dtype, dim3 g, hipStream_t stream) {
  dim3 blk(NT * KVS);
  if (D == 128) {
    if (o_dtype == RA_BF16) hipLaunchKernelGGL((attn_bf16_kernel<128, OutBf16, KVS, PAIR, DBG>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<128, OutF32, KVS, PAIR, DBG>), g, blk, 0, stream, a);
  } else {
    if (o_dtype == RA_BF16) hipLaunchKernelGGL((attn_bf16_kernel<64, OutBf16, KVS, PAIR, DBG>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<64, OutF32, KVS, PAIR, DBG>), g, blk, 0, stream, a);
  }
}

// The counting copy is chosen only when a debug buffer is passed; the layout choice is the same.
template <int KVS, int PAIR>
static void launch(const AttnArgs& a, int D, int o_dtype, dim3 g, hipStream_t stream) {
  if (a.dbg_counts) launch_dbg<KVS, PAIR, 1>(a, D, o_dtype, g, stream);
  else launch_dbg<KVS, PAIR, 0>(a, D, o_dtype, g, stream);
}

hipError_t launch_attn_bf16(const AttnArgs& a, int D, int o_dtype, hipStream_t stream) {
  const int n_qt = (a.Sq + BM - 1) / BM;
  const int64_t grid = (int64_t)n_qt * a.B * a.H;
  if (grid == 0) return hipSuccess;
  // Key split when one workgroup per query tile leaves CUs with fewer than two workgroups.
  const int mode = kv_split_override();
  if constexpr (QB == 1) {  // the split layout merges one 32-row block per wave
    if (mode > 0 || (mode == 0 && grid < 2 * (int64_t)device_cus())) {
      launch<2, 0>(a, D, o_dtype, dim3((unsigned)grid), stream);
      return hipGetLastError();
    }
  }
  // Pair query tiles (n_qt-1-p, p) on striped shares when the halved grid still fills every CU
  // twice; RA_PAIR_TILES=always pairs any causal call with two or more query tiles.
  const int64_t pairs = (int64_t)(n_qt + 1) / 2 * a.B * a.H;
  const int pmode = pair_override();
  const bool pair = a.causal && n_qt >= 2 &&
                    (pmode > 0 || (pmode == 0 && a.kv_assign == RA_STRIPED && pairs >= 2 * (int64_t)device_cus()));
  if (pair) {
    // Short shares (a few dozen key tiles per step) keep the paired workgroups of a head on the
    // same key tiles better with groups of 8 tiles; long shares with groups of 32.
    const int gmode = pair_group_override();
    if (gmode < 0 || (gmode == 0 && a.Sk <= RA_ATTN_SHORT_SHARE)) launch<1, 2>(a, D, o_dtype, dim3((unsigned)pairs), stream);
    else launch<1, 1>(a, D, o_dtype, dim3((unsigned)pairs), stream);
    return hipGetLastError();
  }
  launch<1, 0>(a, D, o_dtype, dim3((unsigned)grid), stream);
  return hipGetLastError();
}

}  // namespace ra
