// Backward pass of the per-device ring attention: dQ of the local Q share and, for every KV
// share of the ring, dK and dV of that share's keys from this share's queries (what would
// travel back around the ring to the share's owner).
//
// The pages train with ring attention ([Digest] "从 Ring Attention 到 DeepSpeed Ulysses，再到
// USP 统一框架", §3.1-§3.4) but print no backward formulas; the kernels differentiate the
// forward definition (softmax of the scaled, masked logits times V, §2) with the saved
// row LSE:
//     P = exp(s - LSE),  Delta = rowsum(dO * O),  dS = P (dO V^T - Delta),
//     dQ = scale dS K,   dK = scale dS^T Q,       dV = P^T dO.
//
// Three launches, bf16 inputs, fp32 gradients:
//  * delta_kernel   Delta [B, H, S] = sum over d of O * dO, and the LSE in log2 units (HBM-bound);
//  * dq_kernel      query-stationary like the forward: a workgroup of 4 wave64s owns 128
//                   query rows of one (batch, head) and walks the visible K/V tiles of every
//                   step; per 64-key tile it forms S^T = K Q^T and dP^T = V dO^T with
//                   v_mfma_f32_32x32x16_bf16 (lane = query row), P^T and dS^T in registers,
//                   and dQ^T += K^T dS^T with K read transposed (ds_read_b64_tr_b16);
//  * dkdv_kernel    key-stationary: a workgroup owns 128 keys of one (batch, KV head, share)
//                   with K in registers and V in LDS (255 registers per lane, so two
//                   workgroups share a CU), and walks the query tiles that can see them
//                   for every query head of the KV head's group; per 64-query tile
//                   S = Q K^T and dP = dO V^T (lane = key), then dV^T += dO^T P and
//                   dK^T += Q^T dS with Q and dO read transposed. No atomics: each workgroup
//                   owns its keys' gradients.
// Tiles go HBM -> LDS with buffer_load ... lds through buffer resources covering the valid rows
// only (rows past the end read as zeros); 16-byte chunks of each LDS row are XOR-permuted by
// the row so that 128-bit row reads stay conflict-free.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "ra_internal.h"

namespace ra {
namespace {

// Row terms (Delta, then the log2 LSE) of the allocation-free entry point (ra_ring_share_bwd_noalloc): every call
// on a device uses that device's copy of this array. Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol): it passes the device address
// from bwd_scratch().
static __device__ __attribute__((aligned(256))) float scratch[RA_BWD_NOALLOC_MAX_BYTES / 4];

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;        // waves per workgroup
constexpr int NT = 64 * NW;  // threads per workgroup
constexpr int QT = 128;      // dq_kernel: query rows per workgroup (32 per wave)
constexpr int KT = 128;      // dkdv_kernel: keys per workgroup (32 per wave)
constexpr int BT = 64;       // rows of a streamed tile (keys in dq_kernel, queries in dkdv_kernel)
static_assert(KT % BT == 0, "the dK/dV kernel stages its V rows as whole tiles");
#ifndef RA_DQ_SCHED
#define RA_DQ_SCHED 1        // dQ kernel: interleave each chunk's dQ MFMAs with the next chunk's dS work
#endif
#ifndef RA_DQ_SCHED_FIRST
#define RA_DQ_SCHED_FIRST 36  // vector ops of the first chunk ahead of the first dQ MFMA
#endif
#ifndef RA_DKDV_WG_PER_CU
#define RA_DKDV_WG_PER_CU 2  // dK/dV workgroups resident per CU (registers per lane: 512 / this)
#endif
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer: untyped dwords, reads past the end give 0

template <int D>
struct Lay {
  static constexpr int ROWB = D * 2;              // bytes per LDS row
  static constexpr int SPR = D / 8;               // 16-byte chunks per row
  static constexpr int RPB = 256 / ROWB;          // rows per 256-byte sweep of the banks
  static constexpr int ELEMS = BT * D;            // one tile
  static constexpr int RPC = 64 / SPR;            // rows per 1 KB copy instruction
  static constexpr int DMA = BT * ROWB / 1024 / NW;  // copies per wave per tile
  static_assert(BT * ROWB % (1024 * NW) == 0, "tile copy must divide over the waves");
  // physical chunk of logical chunk c in row r is c ^ swz(r)
  static __device__ constexpr int swz(int r) { return (r / RPB) & (SPR - 1); }
};

__device__ inline s16x4 read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource over `rows` rows of `rowb` bytes starting at `base`.
__device__ inline __amdgpu_buffer_rsrc_t rows_rsrc(const char* base, int rows, uint32_t rowb) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)((uint32_t)rows * rowb), kBufferWord3);
}

// Copy a BT-row tile (row stride `rowb` bytes in HBM, D elements used per row) into LDS `tile`.
template <int D>
__device__ inline void copy_tile(__amdgpu_buffer_rsrc_t r, __bf16* tile, uint32_t rowb, int wave, int lane) {
  using L = Lay<D>;
  int lr = lane / L::SPR, lc = lane % L::SPR;
  asm volatile("" : "+v"(lr), "+v"(lc));  // formed at each copy: kept live they would cost registers
  const uint32_t lb = __umul24((uint32_t)lr, rowb);  // rows are below 2^24 bytes (checked on the host)
#pragma unroll
  for (int i = 0; i < L::DMA; ++i) {
    const int row0 = (wave * L::DMA + i) * L::RPC;  // wave-uniform: the copy's scalar offset
    const uint32_t off = lb + (uint32_t)((lc ^ L::swz(row0 + lr)) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(tile + (wave * L::DMA + i) * 512),
                                             16, off, (uint32_t)row0 * rowb, 0, 0);
  }
}

// Per-lane byte offsets for reading a tile (a) as MFMA A-operand rows, 32 rows from `row0`:
// lane l reads row l%32, logical chunk 2ks + l/32; (b) transposed, as an A operand whose k
// index runs over 16 tile rows: two ds_read_b64_tr_b16 (rows r..r+3 and r+8..r+11 of each 16)
// give the 8 rows in the order a 32x32 accumulator hands its registers to a B operand.
template <int D>
struct Offsets {
  using L = Lay<D>;
  int row[D / 16];
  int tr_lo[D / 32], tr_hi[D / 32];
  __device__ explicit Offsets(int lane) {
    const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) row[ks] = l32 * L::ROWB + (((2 * ks + hh) ^ L::swz(l32)) * 16);
    const int g16 = lane >> 4, jj = lane & 15;
    const int vr = 4 * (g16 >> 1) + (jj >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = 4 * db + 2 * (g16 & 1) + ((jj & 3) >> 1);
      tr_lo[db] = vr * L::ROWB + ((c ^ L::swz(vr)) * 16) + (jj & 1) * 8;
      tr_hi[db] = (vr + 8) * L::ROWB + ((c ^ L::swz(vr + 8)) * 16) + (jj & 1) * 8;
    }
  }
};

// A operand (32 d-rows x 16 tile rows) of tile rows [r0, r0+16), head-dim block db.
template <int D>
__device__ inline bf16x8 read_t(const __bf16* tile, const Offsets<D>& of, int db, int r0) {
  const char* p = (const char*)tile + r0 * Lay<D>::ROWB;
  const s16x4 lo = read_tr(p + of.tr_lo[db]);
  const s16x4 hi = read_tr(p + of.tr_hi[db]);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand (32 tile rows from r0 x 16 d) for head-dim step ks.
template <int D>
__device__ inline bf16x8 read_r(const __bf16* tile, const Offsets<D>& of, int ks, int r0) {
  return *(const bf16x8*)((const char*)tile + r0 * Lay<D>::ROWB + of.row[ks]);
}

// Also stores the LSE in log2 units (lse2 = LSE * log2 e; +inf for a row with no visible key,
// so that its weights come out 0), the form the dK/dV kernel takes its weights against.
// D/8 consecutive lanes share one (b, s, h) row, 16 bytes of O and of dO each, so every load
// instruction of a wave reads whole consecutive rows; the row's partial sums meet by shuffles.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dout,
                                                    const float* __restrict__ lse, float* __restrict__ delta,
                                                    float* __restrict__ lse2, int64_t B, int64_t S, int64_t H) {
  constexpr int LPR = D / 8;      // lanes per row
  constexpr int RPB = 256 / LPR;  // rows per workgroup
  const int64_t rows = B * S * H;
  const int c = threadIdx.x % LPR;
  // workgroup-uniform loop over row groups (every lane takes part in the shuffles)
  for (int64_t base = (int64_t)blockIdx.x * RPB; base < rows; base += (int64_t)gridDim.x * RPB) {
    const int64_t u = base + threadIdx.x / LPR;  // (b, s, h) row
    float acc = 0.f;
    if (u < rows) {
      const bf16x8 x = ((const bf16x8*)(o + u * D))[c];
      const bf16x8 y = ((const bf16x8*)(dout + u * D))[c];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (u < rows && c == 0) {
      const int64_t h = u % H, s = (u / H) % S, b = u / (H * S);
      const int64_t r = (b * H + h) * S + s;
      delta[r] = acc;
      const float ln = lse[r];
      lse2[r] = ln == -INFINITY ? INFINITY : ln * kLog2e;
    }
  }
}

template <int D>
__global__ __launch_bounds__(NT, 2) void dq_kernel(const BwdArgs a) {
  using L = Lay<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 k_l[2][L::ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 v_l[2][L::ELEMS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int nbh = a.B * a.H;
  const int n_qt = (a.Sq + QT - 1) / QT;
  const int bh = blockIdx.x % nbh;
  const int qt = n_qt - 1 - (int)(blockIdx.x / nbh);  // heaviest query tile first
  const int b = bh / a.H, h = bh % a.H, hk = h / (a.H / a.Hkv);
  const int q0 = qt * QT, w0 = q0 + wave * 32, row = w0 + l32;
  const bool wave_live = w0 < a.Sq;
  const int rq = min(row, a.Sq - 1);
  const int64_t rs = (int64_t)a.H * D, rs_kv = (int64_t)a.Hkv * D;
  const uint32_t rowb_kv = (uint32_t)rs_kv * 2;
  const float sl2 = a.scale * kLog2e;

  bf16x8 qreg[D / 16], doreg[D / 16];
  {
    const int64_t off = ((int64_t)b * a.Sq + rq) * rs + (int64_t)h * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qreg[ks] = *(const bf16x8*)((const __bf16*)a.q + off + ks * 16);
      doreg[ks] = *(const bf16x8*)((const __bf16*)a.dout + off + ks * 16);
    }
  }
  const int64_t srow = ((int64_t)b * a.H + h) * a.Sq + rq;
  const float lse_n = a.lse[srow];
  const float lse2 = lse_n == -INFINITY ? INFINITY : lse_n * kLog2e;  // no visible key: P = 0
  const float dlt = a.delta[srow];

  int32_t wg_qmin = 0, wg_qmax = 0, w_qmin = 0, my_qpos = -1;
  if (a.causal) {
    wg_qmin = pos_of(a.qpos, q0);
    wg_qmax = pos_of(a.qpos, min(q0 + QT, a.Sq) - 1);
    if (wave_live) w_qmin = pos_of(a.qpos, w0);
    if (row < a.Sq) my_qpos = pos_of(a.qpos, row);
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;
  const Offsets<D> of(lane);

  for (int s = 0; s < a.nsteps; ++s) {
    Pos kvp = make_pos(a.kv_assign, a.kv_world, a.kv_rank[s], a.kv_len);
    int nt = (a.Sk + BT - 1) / BT, nf = a.Sk / BT;
    if (a.causal) {
      nt = (clamp32(count_le(kvp, wg_qmax), 0, a.Sk) + BT - 1) / BT;
      nf = clamp32(count_le(kvp, wg_qmin), 0, a.Sk) / BT;
    }
    if (nt == 0) continue;
    const char* kbase = (const char*)a.k[s] + ((int64_t)b * a.Sk * rs_kv + (int64_t)hk * D) * 2;
    const char* vbase = (const char*)a.v[s] + ((int64_t)b * a.Sk * rs_kv + (int64_t)hk * D) * 2;
    auto fetch = [&](int t, int st) {
      const int rows = min(BT, a.Sk - t * BT);
      copy_tile<D>(rows_rsrc(kbase + (int64_t)t * BT * rowb_kv, rows, rowb_kv), k_l[st], rowb_kv, wave, lane);
      copy_tile<D>(rows_rsrc(vbase + (int64_t)t * BT * rowb_kv, rows, rowb_kv), v_l[st], rowb_kv, wave, lane);
    };
    fetch(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      const int st = t & 1;
      if (t + 1 < nt) fetch(t + 1, st ^ 1);  // stage st^1 was last read before the previous barrier
      if (wave_live) {
        const __bf16* kt = k_l[st];
        const __bf16* vt = v_l[st];
        f32x16 sc[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f, dp[kb][r] = 0.f;
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_r<D>(kt, of, ks, kb * 32), qreg[ks], sc[kb], 0, 0, 0);
            dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_r<D>(vt, of, ks, kb * 32), doreg[ks], dp[kb], 0, 0, 0);
          }
        }
        // visibility: keys of a share visible to a query form a prefix of the share
        const int key0 = t * BT;
        bool masked = key0 + BT > a.Sk;
        if (a.causal) masked = masked || (t >= nf && w_qmin < pos_of(kvp, min(key0 + BT, a.Sk) - 1));
        if (masked) {
          // a tile on the causal boundary or the ragged end: the scores of keys past the row's
          // visible prefix become -inf (weight 0), so the weights below need no mask and no
          // branch per score
          const int lim = (a.causal ? clamp32(count_le(kvp, my_qpos), 0, a.Sk) : a.Sk) - key0 - hh * 4;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
              sc[kb][r] = off < lim ? sc[kb][r] : -INFINITY;
            }
        }
        // dS of each 16-key chunk, then dQ^T += K^T dS^T for its keys (one MFMA per 32 head-dim
        // rows); the MFMAs of a chunk issue between the vector work of the next one
        bf16x8 dsb[4];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kb = ch >> 1, r = (ch & 1) * 8 + e;
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], sl2, -lse2));
            dsb[ch][e] = (__bf16)(p * (dp[kb][r] - dlt));
          }
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
            dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_t<D>(kt, of, db, ch * 16), dsb[ch], dq[db], 0, 0, 0);
        }
#if RA_DQ_SCHED
        __builtin_amdgcn_sched_group_barrier(0x002, RA_DQ_SCHED_FIRST, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 4 * (D / 32); ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, RA_DQ_SCHED_FIRST / (D / 32), 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#endif
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  if (row < a.Sq) {
    const int64_t out = (((int64_t)b * a.Sq + row) * a.H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dq[db][g * 4 + e] * a.scale;
        *(f32x4*)(a.dq + out + db * 32 + g * 8 + hh * 4) = x;
      }
  }
}

template <int D>
__global__ __launch_bounds__(NT, RA_DKDV_WG_PER_CU) void dkdv_kernel(const BwdArgs a) {
  using L = Lay<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 v_l[KT * D];       // V of the workgroup's keys
  __shared__ __attribute__((aligned(1024))) __bf16 q_l[L::ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 o_l[L::ELEMS];     // the dO tile
  __shared__ __attribute__((aligned(256))) float lse_l[BT];
  __shared__ __attribute__((aligned(256))) float dlt_l[BT];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int n_kt = (a.Sk + KT - 1) / KT;
  int idx = blockIdx.x;
  const int kt = idx % n_kt;
  idx /= n_kt;
  const int hk = idx % a.Hkv;
  idx /= a.Hkv;
  const int b = idx % a.B;
  const int s = idx / a.B;  // step of the call: KV share a.kv_rank[s]
  const int group = a.H / a.Hkv;
  const int k0 = kt * KT, wk0 = k0 + wave * 32, key = wk0 + l32;
  const bool wave_live = wk0 < a.Sk;
  const int rk = min(key, a.Sk - 1);
  const int64_t rs = (int64_t)a.H * D, rs_kv = (int64_t)a.Hkv * D;
  const uint32_t rowb_q = (uint32_t)rs * 2, rowb_kv = (uint32_t)rs_kv * 2;
  const float sl2 = a.scale * kLog2e;

  // K of this lane's key in registers (B operand of S = Q K^T); V of the workgroup's KT keys in
  // LDS (B operand of dP = dO V^T, read per use), laid out as two consecutive swizzled tiles.
  bf16x8 kreg[D / 16];
  {
    const int64_t off = ((int64_t)b * a.Sk + rk) * rs_kv + (int64_t)hk * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kreg[ks] = *(const bf16x8*)((const __bf16*)a.k[s] + off + ks * 16);
    const char* vbase = (const char*)a.v[s] + ((int64_t)b * a.Sk * rs_kv + (int64_t)hk * D) * 2;
#pragma unroll
    for (int half = 0; half < KT / BT; ++half) {
      const int r0 = k0 + half * BT;
      const int rows = max(0, min(BT, a.Sk - r0));
      copy_tile<D>(rows_rsrc(vbase + (int64_t)r0 * rowb_kv, rows, rowb_kv), v_l + half * L::ELEMS, rowb_kv, wave, lane);
    }
  }
  // Queries see a key iff their position is at least the key's: a suffix of the Q share.
  const Pos kvp = make_pos(a.kv_assign, a.kv_world, a.kv_rank[s], a.kv_len);
  int qfirst = 0, w_qfirst_max = 0, qt0 = 0;
  if (a.causal) {
    qfirst = clamp32(count_le(a.qpos, pos_of(kvp, rk) - 1), 0, a.Sq);             // this lane's key
    if (wave_live) w_qfirst_max = clamp32(count_le(a.qpos, pos_of(kvp, min(wk0 + 31, a.Sk - 1)) - 1), 0, a.Sq);
    qt0 = clamp32(count_le(a.qpos, pos_of(kvp, k0) - 1), 0, a.Sq) / BT;  // the workgroup's first key
  }
  const int n_qt = (a.Sq + BT - 1) / BT;

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[db][r] = 0.f, dv[db][r] = 0.f;
  const Offsets<D> of(lane);

  for (int g = 0; g < group; ++g) {
    const int h = hk * group + g;
    const char* qbase = (const char*)a.q + ((int64_t)b * a.Sq * rs + (int64_t)h * D) * 2;
    const char* obase = (const char*)a.dout + ((int64_t)b * a.Sq * rs + (int64_t)h * D) * 2;
    const int64_t srow0 = ((int64_t)b * a.H + h) * a.Sq;
    // Query tiles from the last one down: every key tile's walk ends at the last query tile, so
    // workgroups of a head that start together read the same Q and dO tiles together.
    for (int qt = n_qt - 1; qt >= qt0; --qt) {
      const int q0 = qt * BT;
      const int rows = min(BT, a.Sq - q0);
      // Q and dO rows by 16-byte LDS DMA over all waves; LSE (natural log) and Delta by 4-byte
      // LDS DMA, one wave each (lane l lands at word l; rows past the share's end read as 0).
      copy_tile<D>(rows_rsrc(qbase + (int64_t)q0 * rowb_q, rows, rowb_q), q_l, rowb_q, wave, lane);
      copy_tile<D>(rows_rsrc(obase + (int64_t)q0 * rowb_q, rows, rowb_q), o_l, rowb_q, wave, lane);
      if (wave < 2) {
        const float* src = (wave == 0 ? a.lse2 : a.delta) + srow0 + q0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc((const char*)src, rows, 4),
                                                 (__attribute__((address_space(3))) void*)(wave == 0 ? lse_l : dlt_l),
                                                 4, (uint32_t)lane * 4, 0, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (wave_live) {
        const bool masked = q0 + BT > a.Sq || (a.causal && q0 < w_qfirst_max);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {  // 32 queries at a time
          f32x16 sc, dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[r] = 0.f, dp[r] = 0.f;
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_r<D>(q_l, of, ks, qb * 32), kreg[ks], sc, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_r<D>(o_l, of, ks, qb * 32),
                                                         read_r<D>(v_l, of, ks, wave * 32), dp, 0, 0, 0);
          }
          // register r of lane l holds query qb*32 + 8*(r/4) + 4*(l/32) + r%4 and key l%32
          if (masked) {
            // scores of pairs the key does not see (or of rows past the share) become -inf, so
            // their weights below come out 0 with no branch per score (a guarded exp2 compiles
            // to a branch on the lane mask for every score)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int iq = q0 + qb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);  // local query index
              sc[r] = ((iq < a.Sq) & (!a.causal | (iq >= qfirst))) ? sc[r] : -INFINITY;
            }
          }
          bf16x8 pb[2], dsb[2];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 ls = *(const f32x4*)(lse_l + qb * 32 + 8 * j + 4 * hh);
            const f32x4 dl = *(const f32x4*)(dlt_l + qb * 32 + 8 * j + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * j + e;
              // LSE is finite, or +inf for a row with no visible key: the weight is 0 there too
              const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], sl2, -ls[e]));
              pb[r >> 3][r & 7] = (__bf16)p;
              dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dl[e]));
            }
          }
          // dV^T += dO^T P and dK^T += Q^T dS, 16 queries per MFMA
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
              dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_t<D>(o_l, of, db, qb * 32 + c * 16), pb[c], dv[db], 0, 0, 0);
              dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_t<D>(q_l, of, db, qb * 32 + c * 16), dsb[c], dk[db], 0, 0, 0);
            }
        }
      }
      __syncthreads();  // every wave is done with this tile before the next copy
    }
  }
  // A workgroup whose keys no query sees ran no tile: let its V copies land before it exits.
  __builtin_amdgcn_s_waitcnt(0);

  if (key < a.Sk) {
    const int64_t out = (((int64_t)b * a.Sk + key) * a.Hkv + hk) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 x, y;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dk[db][g4 * 4 + e] * a.scale, y[e] = dv[db][g4 * 4 + e];
        *(f32x4*)(a.dk[s] + out + db * 32 + g4 * 8 + hh * 4) = x;
        *(f32x4*)(a.dv[s] + out + db * 32 + g4 * 8 + hh * 4) = y;
      }
  }
}

}  // namespace

hipError_t bwd_scratch(float** out) {
  // The array's device address, looked up once per device (with that device current) and kept.
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = (float*)p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_attn_bwd(const BwdArgs& a, int D, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Sq * a.H;
  if (rows == 0) return hipSuccess;
  const int64_t rpb = 256 / (D / 8);  // rows per delta_kernel workgroup and pass
  const unsigned g_delta = (unsigned)std::min<int64_t>((rows + rpb - 1) / rpb, (int64_t)1 << 20);
  if (D == 128)
    hipLaunchKernelGGL(delta_kernel<128>, dim3(g_delta), dim3(256), 0, stream,
                       (const __bf16*)a.o, (const __bf16*)a.dout, a.lse, a.delta, a.lse2, (int64_t)a.B, (int64_t)a.Sq,
                       (int64_t)a.H);
  else
    hipLaunchKernelGGL(delta_kernel<64>, dim3(g_delta), dim3(256), 0, stream,
                       (const __bf16*)a.o, (const __bf16*)a.dout, a.lse, a.delta, a.lse2, (int64_t)a.B, (int64_t)a.Sq,
                       (int64_t)a.H);
  const int64_t gq = (int64_t)((a.Sq + QT - 1) / QT) * a.B * a.H;
  const int64_t gk = (int64_t)((a.Sk + KT - 1) / KT) * a.B * a.Hkv * a.nsteps;
  if (D == 128) {
    hipLaunchKernelGGL(dq_kernel<128>, dim3((unsigned)gq), dim3(NT), 0, stream, a);
    if (gk) hipLaunchKernelGGL(dkdv_kernel<128>, dim3((unsigned)gk), dim3(NT), 0, stream, a);
  } else {
    hipLaunchKernelGGL(dq_kernel<64>, dim3((unsigned)gq), dim3(NT), 0, stream, a);
    if (gk) hipLaunchKernelGGL(dkdv_kernel<64>, dim3((unsigned)gk), dim3(NT), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ra
