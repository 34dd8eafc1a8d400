// Internal declarations shared by the host API layer and the gfx950 kernels.
//
// Position arithmetic ([Digest] = "从 Ring Attention 到 DeepSpeed Ulysses，再到 USP
// 统一框架", jsqmd.com): contiguous split (§3.4 and the §4 listing), striped split (§4),
// zigzag split (§6 item 1). The same functions serve the host planner, the debug hooks and
// the kernels' tile classification and masks, so all three agree by construction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ra.h"

namespace ra {

// Position rule of one share: local row i -> global token position. Global lengths are
// validated to stay below 2^31, so positions and counts fit 32-bit integers.
struct Pos {
  int32_t assign;  // ra_assign
  int32_t world;
  int32_t rank;
  int32_t share;   // rows per share, L / N
  int32_t chunk;   // zigzag chunk length, L / (2N) (unused otherwise)
};

__host__ __device__ inline Pos make_pos(int assign, int world, int rank, int64_t len) {
  Pos p;
  p.assign = assign;
  p.world = world;
  p.rank = rank;
  p.share = (int32_t)(len / world);
  p.chunk = (int32_t)(len / (2 * (int64_t)world));
  return p;
}

__host__ __device__ inline int32_t pos_of(const Pos& p, int32_t i) {
  if (p.assign == RA_STRIPED) return i * p.world + p.rank;
  if (p.assign == RA_ZIGZAG)
    return i < p.chunk ? p.rank * p.chunk + i : (2 * p.world - 1 - p.rank) * p.chunk + (i - p.chunk);
  return p.rank * p.share + i;  // RA_CONTIGUOUS
}

__host__ __device__ inline int32_t clamp32(int32_t x, int32_t lo, int32_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

__host__ __device__ inline int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Number of local rows whose global position is <= x. Positions increase with the local
// row index under all three assignments, so these rows are a prefix of the share.
__host__ __device__ inline int32_t count_le(const Pos& p, int32_t x) {
  if (p.assign == RA_STRIPED) {
    if (x < p.rank) return 0;
    return clamp32((x - p.rank) / p.world + 1, 0, p.share);
  }
  if (p.assign == RA_ZIGZAG) {
    const int32_t lo = clamp32(x - p.rank * p.chunk + 1, 0, p.chunk);
    const int32_t hi = clamp32(x - (2 * p.world - 1 - p.rank) * p.chunk + 1, 0, p.chunk);
    return lo + hi;
  }
  return clamp32(x - p.rank * p.share + 1, 0, p.share);
}

// Causal visibility by global position, diagonal included ([Digest] §3.4 causal matrix).
__host__ __device__ inline bool visible(int32_t qpos, int32_t kpos) { return kpos <= qpos; }

constexpr int kMaxSteps = RA_MAX_WORLD;

// Arguments of the attention kernels. Steps are already in ring order: entry s is the KV
// share visited at step s and kv_rank[s] is the rank that share belongs to.
struct AttnArgs {
  const void* q;
  const void* k[kMaxSteps];
  const void* v[kMaxSteps];
  int32_t kv_rank[kMaxSteps];
  void* o;
  float* lse;
  float* ws_o;   // running state (may be null when neither loaded nor stored):
  double* ws_m;  // un-normalised O in fp32, running max and running sum in fp64 slots
  double* ws_l;
  int32_t B, H, Sq, Sk;
  int32_t Hkv;          // KV heads (divides H): query head h reads KV head h / (H / Hkv)
  int32_t nsteps;
  int32_t causal;
  int32_t load_state;
  int32_t store_final;  // 1: write normalised O and LSE; 0: write the running state
  Pos qpos;             // rule for Q rows
  int32_t kv_assign, kv_world;
  int64_t kv_len;       // global length of the KV rule (rank comes from kv_rank[s])
  float scale;          // logit scale (natural units)
  // Debug only (null in every product call): per-wave tile counts of the instrumented kernel,
  // int32 [ceil(Sq/BM), B, H, 8, 2]: for wave slot w (group * waves + wave) the K/V tiles it
  // folded in and on how many of them it evaluated the mask.
  int32_t* dbg_counts;
};

// Arguments of the backward launches (bf16 inputs, fp32 gradients; same layouts as AttnArgs).
struct BwdArgs {
  const void* q;
  const void* o;
  const void* dout;     // dO [B, Sq, H, D]
  const float* lse;     // forward LSE [B, H, Sq] (natural log)
  float* delta;         // workspace [B, H, Sq]: rowsum(dO * O)
  float* lse2;          // workspace [B, H, Sq]: LSE * log2 e (+inf for a row with no visible key)
  float* dq;            // [B, Sq, H, D]
  const void* k[kMaxSteps];
  const void* v[kMaxSteps];
  float* dk[kMaxSteps];  // [B, Sk, Hkv, D] per step's share
  float* dv[kMaxSteps];
  int32_t kv_rank[kMaxSteps];
  int32_t B, H, Hkv, Sq, Sk;
  int32_t nsteps;
  int32_t causal;
  Pos qpos;
  int32_t kv_assign, kv_world;
  int64_t kv_len;
  float scale;
};

// Launchers (return hipError_t of the launch).
hipError_t launch_attn_bwd(const BwdArgs& a, int D, hipStream_t stream);
constexpr int kMaxDevices = 64;
// Device address of the backward's static scratch array on the current device.
hipError_t bwd_scratch(float** out);
hipError_t launch_attn_bf16(const AttnArgs& a, int D, int o_dtype, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs& a, int D, int o_dtype, hipStream_t stream);
hipError_t launch_lse_merge(void* o_acc, float* lse_acc, const void* o_blk, const float* lse_blk,
                            int64_t B, int64_t H, int64_t S, int64_t D, int acc_dtype,
                            int blk_dtype, hipStream_t stream);
constexpr int kMaxPermute = RA_MAX_PERMUTE;  // tensors one permute launch moves
hipError_t launch_permute(const void* const* in, void* const* out, int n_t, int64_t B, int64_t P, int64_t S_loc,
                          int64_t H, int64_t D, int esize, int dst_rank, int inverse, hipStream_t stream);
hipError_t launch_debug_positions(Pos p, int64_t n, int64_t* out, hipStream_t stream);
hipError_t launch_debug_mask(Pos q, Pos kv, int64_t Sq, int64_t Sk, uint8_t* out,
                             hipStream_t stream);

// Tile shape of the bf16 MFMA kernel: QB blocks of 32 query rows per wave64.
#ifndef RA_ATTN_WAVES
#define RA_ATTN_WAVES 4
#endif
#ifndef RA_ATTN_QB
#define RA_ATTN_QB 1
#endif
constexpr int kBf16BlockM = 32 * RA_ATTN_QB * RA_ATTN_WAVES;
#ifndef RA_ATTN_BN
#define RA_ATTN_BN 64
#endif
constexpr int kBf16BlockN = RA_ATTN_BN;
// Tile shape of the fp32 kernel.
constexpr int kF32BlockM = 64;
constexpr int kF32BlockN = 32;

}  // namespace ra
