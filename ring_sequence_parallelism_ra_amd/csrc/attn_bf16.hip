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
#ifndef RA_ATTN_WAVES_PER_SIMD
#define RA_ATTN_WAVES_PER_SIMD 2      // occupancy target: 256 VGPRs per wave at 2, 512 at 1
#endif

constexpr int TG = RA_ATTN_TILE_GROUP;

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
template <int D, class Out, int KVS>
__global__ __launch_bounds__(NT * KVS, QB == 1 ? RA_ATTN_WAVES_PER_SIMD : 1) void attn_bf16_kernel(const AttnArgs a) {
  using C = Cfg<D>;
  static_assert(KVS == 1 || (KVS == 2 && QB == 1), "the key split merges one 32-row block per wave");
  // The two stages of K and V are four distinct LDS objects: the copies into one stage and the
  // reads of the other can then be told apart, so no wait for in-flight copies is inserted
  // before the reads.
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds0[C::ELEMS * KVS];
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds1[C::ELEMS * KVS];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds0[C::ELEMS * KVS];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds1[C::ELEMS * KVS];

  const int tid = threadIdx.x;
  const int wave_wg = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep in SGPRs
  const int grp = KVS == 1 ? 0 : wave_wg / RA_ATTN_WAVES;        // key-split group
  const int wave = KVS == 1 ? wave_wg : wave_wg % RA_ATTN_WAVES;  // wave within the group
  const int goff = grp * C::ELEMS;                                // the group's LDS tiles
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int nbh = a.B * a.H;
  const int n_qt = (a.Sq + BM - 1) / BM;
  const int bh = blockIdx.x % nbh;
  const int qt = n_qt - 1 - (int)(blockIdx.x / nbh);  // heaviest (latest) query tile first
  const int b = bh / a.H;
  // Consecutive workgroups go to the 8 XCDs in turn, so head (bh mod H) runs on XCD
  // (bh mod 8) when 8 divides H. With grouped KV heads the heads are renumbered so that each
  // XCD takes a contiguous run of H/8 heads: the query heads sharing a KV head then share one
  // XCD's L2 instead of each XCD reading every KV head.
  const int hr = bh % a.H;
  const int h = (a.Hkv < a.H && a.H % 8 == 0) ? (hr % 8) * (a.H / 8) + hr / 8 : hr;
  const int q0 = qt * BM;
  const int w0 = q0 + wave * WR;  // first row of this wave; block qb owns rows w0+32qb ..
  const bool wave_live = w0 < a.Sq;
  const int64_t rs = (int64_t)a.H * D;       // elements between consecutive Q/O sequence rows
  const int64_t rs_kv = (int64_t)a.Hkv * D;  // ... and K/V rows
  const int hk = h / (a.H / a.Hkv);          // the KV head this query head reads (GQA/MQA)
  const float sl2 = a.scale * kLog2e;
  auto row_of = [&](int qb) { return w0 + 32 * qb + l32; };

  // ---- Q rows of this wave as B operands (k = head dim), resident for the whole kernel.
  bf16x8 qreg[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qr = min(row_of(qb), a.Sq - 1);
    const __bf16* qp = (const __bf16*)a.q + ((int64_t)b * a.Sq + qr) * rs + (int64_t)h * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qreg[qb][ks] = *(const bf16x8*)(qp + ks * 16);
  }

  // ---- positions of the workgroup's, the wave's and this lane's query rows.
  int32_t wg_qmin = 0, wg_qmax = 0, w_qmin = 0, my_qpos[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) my_qpos[qb] = -1;
  if (a.causal) {
    wg_qmin = pos_of(a.qpos, q0);
    wg_qmax = pos_of(a.qpos, min(q0 + BM, a.Sq) - 1);
    if (wave_live) w_qmin = pos_of(a.qpos, w0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      if (row_of(qb) < a.Sq) my_qpos[qb] = pos_of(a.qpos, row_of(qb));
  }

  // ---- running state per row block: m (log2 domain), l (this lane half's keys), O^T.
  float m_run[QB], l_run[QB];
  f32x16 oacc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
  }

  auto state_row = [&](int qb) { return ((int64_t)b * a.H + h) * a.Sq + row_of(qb); };    // [B, H, S]
  auto out_row = [&](int qb) { return (((int64_t)b * a.Sq + row_of(qb)) * a.H + h) * D; };  // [B, S, H, D]
  if (a.load_state && grp == 0) {  // a split workgroup resumes in group 0 only
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (row_of(qb) >= a.Sq) continue;
      m_run[qb] = (float)a.ws_m[state_row(qb)];  // stored from this kernel's own fp32 values: exact
      l_run[qb] = hh == 0 ? (float)a.ws_l[state_row(qb)] : 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x = *(const f32x4*)(a.ws_o + out_row(qb) + db * 32 + g * 8 + hh * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[qb][db][g * 4 + e] = x[e];
        }
    }
  }

  // ---- the (step, tile) sequence this workgroup visits. Tiles are taken in groups of TG
  // consecutive tiles, round-robin over the call's steps: tiles [0, TG) of every step (in step
  // order), then tiles [TG, 2 TG) of every step that still has visible tiles, and so on. The
  // fold is order-independent up to rounding. Taking whole shares one after another lets
  // concurrent workgroups of a head drift onto different shares when their visible prefixes
  // differ in length (short shares, e.g. striped ones), and their K/V tiles then miss in L2;
  // the round-robin keeps them on the same tiles. Lane s of every wave describes step s:
  // visible tiles, fully visible tiles, K/V rank, share pointers.
  const Pos kv_rule = make_pos(a.kv_assign, a.kv_world, 0, a.kv_len);  // rank set per step
  const int64_t bh_off = ((int64_t)b * a.Sk * rs_kv + (int64_t)hk * D) * 2;  // bytes to K/V row 0 of (b, hk)
  int st_nt = 0, st_nf = 0, st_rank = 0;
  uint32_t st_k0 = 0, st_k1 = 0, st_v0 = 0, st_v1 = 0;
  for (int s = 0; s < a.nsteps; ++s) {
    if (lane == s) {
      const uint64_t kp = (uint64_t)(uintptr_t)a.k[s] + (uint64_t)bh_off;
      const uint64_t vp = (uint64_t)(uintptr_t)a.v[s] + (uint64_t)bh_off;
      st_rank = a.kv_rank[s];
      st_k0 = (uint32_t)kp, st_k1 = (uint32_t)(kp >> 32);
      st_v0 = (uint32_t)vp, st_v1 = (uint32_t)(vp >> 32);
    }
  }
  if (lane < a.nsteps) {
    if (a.causal) {
      Pos kp = kv_rule;
      kp.rank = st_rank;
      const int32_t cmax = clamp32(count_le(kp, wg_qmax), 0, a.Sk);
      const int32_t cmin = clamp32(count_le(kp, wg_qmin), 0, a.Sk);
      st_nt = (cmax + BN - 1) / BN;
      st_nf = cmin / BN;
    } else {
      st_nt = (a.Sk + BN - 1) / BN;
      st_nf = a.Sk / BN;
    }
  }
  auto set_step = [&](Cursor& c, int s, int t) {
    c.t = t;
    if (s == c.s && c.nt > 0) return;  // same step: nothing to look up
    c.s = s;
    c.nt = __builtin_amdgcn_readlane(st_nt, s);
    c.nf = __builtin_amdgcn_readlane(st_nf, s);
    c.rank = __builtin_amdgcn_readlane(st_rank, s);
    c.kb = (const char*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)st_k1, s) << 32) |
                                    (uint32_t)__builtin_amdgcn_readlane((int)st_k0, s));
    c.vb = (const char*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)st_v1, s) << 32) |
                                    (uint32_t)__builtin_amdgcn_readlane((int)st_v0, s));
  };
  // Move to the next tile; at the end the cursor stays on the last tile (a harmless dummy).
  auto advance = [&](Cursor& c) {
    if ((c.t + 1) % TG != 0 && c.t + 1 < c.nt) {  // inside a group of TG tiles of one step
      ++c.t;
      return;
    }
    const int g0 = c.t / TG * TG;
    const uint64_t later = c.s >= 63 ? 0ull : (~0ull << (c.s + 1));
    const uint64_t same_g = __builtin_amdgcn_ballot_w64(st_nt > g0) & later;
    if (same_g) {
      set_step(c, __builtin_ctzll(same_g), g0);
      return;
    }
    const uint64_t next_g = __builtin_amdgcn_ballot_w64(st_nt > g0 + TG);
    if (next_g) set_step(c, __builtin_ctzll(next_g), g0 + TG);
  };

  // With the key split, each group takes every KVS-th tile of the sequence from its own start.
  auto step = [&](Cursor& c) {
    advance(c);
    if constexpr (KVS == 2) advance(c);
  };

  int total = 0;
  for (int s = 0; s < a.nsteps; ++s) total += __builtin_amdgcn_readlane(st_nt, s);
  Cursor cur = {-1, 0, 0, 0, 0, nullptr, nullptr};
  const uint64_t first = __builtin_amdgcn_ballot_w64(st_nt > 0);
  if (first) set_step(cur, __builtin_ctzll(first), 0);
  if (KVS == 2 && grp == 1) advance(cur);
  // iterations of the loop (the same for every wave: barriers) and tiles of this wave's group
  const int n_iter = KVS == 1 ? total : (total + 1) / 2;
  const int my_tiles = KVS == 1 ? total : (total + 1 - grp) / 2;

  if (total > 0) {
    // Copy one tile of K or V from HBM into an LDS tile. Lane `lane` of copy i of wave w fills
    // 16-byte slot (w*DMA + i)*64 + lane of the tile: row r = (w*DMA + i)*RPC + lane/SPR (RPC rows
    // per copy) and physical chunk lane%SPR, which holds logical chunk (lane%SPR) ^ swizzle(r).
    // The V swizzle depends only on lane/SPR, so one register holds the lane's part of every V
    // offset; the K swizzle also depends on the copy, and its XOR is formed per copy. The copies
    // go through a buffer resource that covers only the tile's valid rows: rows past Sk of a
    // ragged last tile read as zeros.
    constexpr int RPC = 64 / C::SPR;  // rows per copy instruction
    static_assert((RPC / C::RPB) % 4 == 0, "the V swizzle must repeat within one copy");
    const uint32_t rowb = (uint32_t)rs_kv * 2;
    const int lrow = lane / C::SPR, lchunk = lane % C::SPR;
    auto tile_rsrc = [&](const char* share, int t) {
      const int rows = min(BN, a.Sk - t * BN);
      return __builtin_amdgcn_make_buffer_rsrc((void*)(share + (int64_t)t * BN * rowb), (short)0,
                                               (int)((uint32_t)rows * rowb), kBufferWord3);
    };
    auto dma = [&](__amdgpu_buffer_rsrc_t r, __bf16* tile, bool is_k) {
      // Formed here, at each use: kept live across the loop these would cost registers.
      int lr = lrow, lc = lchunk;
      asm volatile("" : "+v"(lr), "+v"(lc));
      const uint32_t lb = (uint32_t)lr * rowb;                          // lane's row in the copy
      const uint32_t vl = lb + (uint32_t)((lc ^ C::v_swz(lr)) * 16);    // V: same for every copy
#pragma unroll
      for (int i = 0; i < C::DMA; ++i) {
        const int row0 = (wave * C::DMA + i) * RPC;  // wave-uniform
        const uint32_t lane_part = is_k ? lb + (uint32_t)((lc ^ C::k_swz(row0 + lr)) * 16) : vl;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(tile + (wave * C::DMA + i) * 512),
                                                 16, (uint32_t)row0 * rowb + lane_part, 0, 0, 0);
      }
    };
    // Lane-constant byte offsets of the swizzled reads (the XOR depends only on the lane).
    int kofs[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kofs[ks] = l32 * C::ROWB + (((2 * ks + hh) ^ C::k_swz(l32)) * 16);
    const int g16 = lane >> 4, jj = lane & 15;
    const int vrow = 4 * (g16 >> 1) + (jj >> 2);  // key of this lane's transposed-read address
    int vofs[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      vofs[db] = vrow * C::ROWB + (((4 * db + 2 * (g16 & 1) + ((jj & 3) >> 1)) ^ C::v_swz(vrow)) * 16) + (jj & 1) * 8;

    // S^T of one tile for every row block of the wave; each K operand read feeds QB MFMAs.
    auto qk = [&](const __bf16* kt, f32x16 (&s)[QB][BN / 32]) {
      const char* kb8 = (const char*)kt;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 ka = *(const bf16x8*)(kb8 + kofs[ks] + kb * 32 * C::ROWB);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][ks], s[qb][kb], 0, 0, 0);
        }
      }
    };

    // Phase A of folding tile `c` (scores in s): causal/ragged mask where the tile needs
    // one, each row's tile max and, where it exceeds the running max, the rescale of O and l.
    // Sets the reference values the tile's weights are taken against.
    auto prepare = [&](const Cursor& c, f32x16 (&s)[QB][BN / 32], float (&base)[QB]) {
      const int key0 = c.t * BN;
      bool masked = key0 + BN > a.Sk;
      Pos kvp = kv_rule;
      kvp.rank = c.rank;
      if (a.causal) masked = masked || (c.t >= c.nf && w_qmin < pos_of(kvp, min(key0 + BN, a.Sk) - 1));
      if (masked) {
        // The keys a query sees form a prefix of the share: mask from its length.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int32_t nvis = a.causal ? clamp32(count_le(kvp, my_qpos[qb]), 0, a.Sk) : a.Sk;
          const int lim = nvis - key0 - hh * 4;  // compared with the lane's key offsets
#pragma unroll
          for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
              s[qb][kb][r] = off < lim ? s[qb][kb][r] : -INFINITY;
            }
        }
      }
      float mc[QB];
      bool any_upd = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mt = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[qb][kb][r]);
        mc[qb] = pair_max(mt) * sl2;
        any_upd = any_upd || (mc[qb] > m_run[qb]);
      }
      if (__any(any_upd)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          // rows that keep their reference value (possibly -inf: no visible key yet) keep O
          const bool upd = mc[qb] > m_run[qb];
          const float alpha = upd ? __builtin_amdgcn_exp2f(m_run[qb] - mc[qb]) : 1.f;
          m_run[qb] = upd ? mc[qb] : m_run[qb];
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) base[qb] = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
    };

    // Phase B, one branch-free block: the weights of the current tile (exp2), O^T += V^T P^T
    // for it, and the next tile's S^T = K Q^T, in four chunks of 16 keys so that the MFMAs of
    // both products are issued between the VALU work of the softmax. Every V and K operand
    // read feeds one MFMA per row block.
    auto fold_and_score = [&](f32x16 (&sc)[QB][BN / 32], const float (&base)[QB], const __bf16* vt,
                              f32x16 (&sn)[QB][BN / 32], const __bf16* kt) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sn[qb][kb][r] = 0.f;
      const char* vt8 = (const char*)vt;
      const char* kt8 = (const char*)kt;
#pragma unroll
      for (int ch = 0; ch < 2 * (BN / 32); ++ch) {
        const int kb = ch >> 1, j = ch & 1;
        bf16x8 pb[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(fmaf(sc[qb][kb][j * 8 + e], sl2, -base[qb]));
            pb[qb][e] = (__bf16)p[e];
          }
          // the chunk's sums as short trees (no long dependency chains through the block)
          l_run[qb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        }
        // O^T += V^T P^T for these 16 keys (one MFMA per 32 head-dim rows), alternating with
        // the next tile's S^T chain for key block kb, head-dim steps j*D/32 .. j*D/32 + D/32-1.
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const char* vp = vt8 + vofs[db] + (kb * 32 + j * 16) * C::ROWB;
          const s16x4 lo = read_tr((const __bf16*)vp);
          const s16x4 hi = read_tr((const __bf16*)(vp + 8 * C::ROWB));
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qb], oacc[qb][db], 0, 0, 0);
          const int ks = j * (D / 32) + db;
          const bf16x8 ka = *(const bf16x8*)(kt8 + kofs[ks] + kb * 32 * C::ROWB);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sn[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][ks], sn[qb][kb], 0, 0, 0);
        }
      }
#if RA_ATTN_SCHED
      // Issue order for the block above: the first chunk's weights, a few operand reads ahead,
      // then after each MFMA a short run of VALU work (the next weights) and the reads for the
      // MFMAs ahead, so LDS latency and the softmax hide under the matrix-core work.
      __builtin_amdgcn_sched_group_barrier(0x002, 28, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, RA_ATTN_SCHED_AHEAD, 0);
      if constexpr (QB == 1) {
#pragma unroll
        for (int i = 0; i < (BN / 32) * (D / 32) * 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, RA_ATTN_SCHED_VALU, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, RA_ATTN_SCHED_VALU, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
        // per 16-key chunk: 2*QB*(D/32) MFMAs, about 28*QB VALU ops and 3*(D/32) LDS reads
#pragma unroll
        for (int ch = 0; ch < 2 * (BN / 32); ++ch)
          sched_chunk<2 * QB * (D / 32), 28 * QB, 3 * (D / 32)>(std::make_integer_sequence<int, 2 * QB * (D / 32)>());
      }
#endif
    };

    // Prologue: K and V of tile 0 and K of tile 1 resident.
    Cursor nx = cur;
    step(nx);
    Cursor k2 = nx;
    step(k2);
    dma(tile_rsrc(cur.kb, cur.t), k_lds0 + goff, true);
    dma(tile_rsrc(cur.vb, cur.t), v_lds0 + goff, false);
    dma(tile_rsrc(nx.kb, nx.t), k_lds1 + goff, true);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed in LDS
    __syncthreads();

    f32x16 s0[QB][BN / 32], s1[QB][BN / 32];
    if (wave_live && (KVS == 1 || my_tiles > 0)) qk(k_lds0 + goff, s0);
    __syncthreads();  // every wave has read K(0) before iteration 0 copies K(2) over it
    // Iteration j (stage sl = j mod 2): LDS holds K(j+1) in stage sl^1 and V(j) in stage sl;
    // registers hold the scores of tile j. It loads K(j+2) into stage sl of K and V(j+1) into
    // stage sl^1 of V, computes the scores of tile j+1 and folds tile j in.
    auto iteration = [&](auto stage, int it, f32x16 (&sc)[QB][BN / 32], f32x16 (&sn)[QB][BN / 32]) {
      constexpr int sl = decltype(stage)::value;
      __bf16* k_fill = (sl ? k_lds1 : k_lds0) + goff;
      __bf16* v_fill = (sl ? v_lds0 : v_lds1) + goff;
      const __bf16* k_read = (sl ? k_lds0 : k_lds1) + goff;
      const __bf16* v_read = (sl ? v_lds1 : v_lds0) + goff;
      dma(tile_rsrc(k2.kb, k2.t), k_fill, true);
      dma(tile_rsrc(nx.vb, nx.t), v_fill, false);
      if (wave_live && (KVS == 1 || it < my_tiles)) {
        float base[QB];
        prepare(cur, sc, base);
        if (RA_ATTN_SETPRIO) __builtin_amdgcn_s_setprio(1);
        fold_and_score(sc, base, v_read, sn, k_read);
        if (RA_ATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
      }
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed in LDS
      __syncthreads();
      cur = nx;
      nx = k2;
      step(k2);
    };
    for (int j = 0; j < n_iter; j += 2) {
      iteration(std::integral_constant<int, 0>(), j, s0, s1);
      if (j + 1 >= n_iter) break;
      iteration(std::integral_constant<int, 1>(), j + 1, s1, s0);
    }
  }

  if constexpr (KVS == 2) {
    // Merge group 1's state into group 0's: wave w of group 1 leaves (m, l, O) in one of the
    // four stage buffers (lane-contiguous words), wave w of group 0 folds it in with the
    // log-sum-exp update (a side that has seen no key contributes nothing).
    float* xs = (float*)(wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1);
    __syncthreads();  // every wave is done with the K/V tiles
    if (grp == 1) {
      xs[lane] = m_run[0];
      xs[64 + lane] = l_run[0];
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[(2 + db * 16 + r) * 64 + lane] = oacc[0][db][r];
    }
    __syncthreads();
    if (grp == 1) return;  // no barrier follows
    const float mb = xs[lane], lb = xs[64 + lane];
    const float m = fmaxf(m_run[0], mb);
    const float fa = m_run[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[0] - m);
    const float fb = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mb - m);
    m_run[0] = m;
    l_run[0] = l_run[0] * fa + lb * fb;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[0][db][r] = oacc[0][db][r] * fa + xs[(2 + db * 16 + r) * 64 + lane] * fb;
  }

  // ---- epilogue
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = pair_sum(l_run[qb]);
    if (row_of(qb) >= a.Sq) continue;
    if (a.store_final) {
      const bool any = l_tot > 0.f;
      const float inv = any ? 1.f / l_tot : 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = oacc[qb][db][g * 4 + e] * inv;
          Out::store4(a.o, out_row(qb) + db * 32 + g * 8 + hh * 4, x);
        }
      if (hh == 0) a.lse[state_row(qb)] = any ? (m_run[qb] + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    } else {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = oacc[qb][db][g * 4 + e];
          *(f32x4*)(a.ws_o + out_row(qb) + db * 32 + g * 8 + hh * 4) = x;
        }
      if (hh == 0) {
        a.ws_m[state_row(qb)] = m_run[qb];
        a.ws_l[state_row(qb)] = l_tot;
      }
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

template <int KVS>
static void launch(const AttnArgs& a, int D, int o_dtype, dim3 g, hipStream_t stream) {
  dim3 blk(NT * KVS);
  if (D == 128) {
    if (o_dtype == RA_BF16) hipLaunchKernelGGL((attn_bf16_kernel<128, OutBf16, KVS>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<128, OutF32, KVS>), g, blk, 0, stream, a);
  } else {
    if (o_dtype == RA_BF16) hipLaunchKernelGGL((attn_bf16_kernel<64, OutBf16, KVS>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<64, OutF32, KVS>), g, blk, 0, stream, a);
  }
}

hipError_t launch_attn_bf16(const AttnArgs& a, int D, int o_dtype, hipStream_t stream) {
  const int n_qt = (a.Sq + BM - 1) / BM;
  const int64_t grid = (int64_t)n_qt * a.B * a.H;
  if (grid == 0) return hipSuccess;
  // Key split when one workgroup per query tile leaves CUs with fewer than two workgroups.
  const int mode = kv_split_override();
  if constexpr (QB == 1) {  // the split layout merges one 32-row block per wave
    if (mode > 0 || (mode == 0 && grid < 2 * (int64_t)device_cus())) {
      launch<2>(a, D, o_dtype, dim3((unsigned)grid), stream);
      return hipGetLastError();
    }
  }
  launch<1>(a, D, o_dtype, dim3((unsigned)grid), stream);
  return hipGetLastError();
}

}  // namespace ra
