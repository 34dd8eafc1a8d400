// Blockwise causal attention with the online-softmax update, bf16 MFMA on gfx950.
//
// What is computed ([Digest] = "从 Ring Attention 到 DeepSpeed Ulysses，再到 USP 统一框架",
// jsqmd.com): softmax(Q K^T / sqrt(d)) V (§2) of one Q share against a sequence of KV
// shares visited in ring order (§3.1, §3.3), each KV tile folded into the running
// (m, l, O) of every query row by the update of §3.2. Masked pairs follow the causal
// matrix of §3.4 by global position.
//
// Mapping onto CDNA4:
//  * A workgroup of 4 wave64s owns BM = 128 query rows of one (batch, head); wave w owns
//    rows 32w .. 32w+31 and lane l owns query row (l mod 32) of its wave.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K tile rows
//    from LDS are the A operand, the wave's Q rows (held in VGPRs for the whole kernel) are
//    the B operand. The 32x32 fp32 result leaves each lane with 16 keys of its own query, so
//    the row max and row sum are in-lane reductions plus one exchange with lane l^32.
//  * O^T += V^T P^T with the same instruction: P^T is the score accumulator converted to
//    bf16 in place (no data movement), V^T comes from LDS, where the V tile is stored
//    transposed with bits 2 and 3 of the key index swapped inside each 16-key group, so
//    that the 8 keys a lane needs are one 16-byte read and match the key order the score
//    accumulator hands to the B operand.
//  * K/V tiles (64 keys) are fetched with 128-bit coalesced global loads into registers
//    one tile ahead and written to the other half of a double-buffered LDS stage, one
//    barrier per tile.
//  * Tiles whose keys are all invisible to the workgroup's rows are never visited: the
//    visible keys of a share form a prefix (positions increase along a share), whose length
//    comes from the position rule. Only tiles straddling the causal boundary or the ragged
//    tail evaluate the mask. Workgroups are launched heaviest query tile first.
//  * Everything in the softmax is kept in the log2 domain (exp2 of scores pre-multiplied by
//    scale*log2 e); LSE is converted back to natural log at the end.
#include <math.h>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kBf16BlockM;   // query rows per workgroup
constexpr int BN = kBf16BlockN;   // keys per tile
constexpr int NT = 256;           // threads per workgroup (4 wave64)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Cfg {
  static constexpr int KS = D + 8;                // K tile row stride in LDS (elements)
  static constexpr int VS = BN + 8;               // V^T tile row stride in LDS
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int KCH = D / 8;               // 16-byte chunks per row
  static constexpr int K_UNITS = BN * KCH;        // (key, chunk) copies per tile
  static constexpr int V_UNITS = (BN / 4) * KCH;  // (4-key group, chunk) copies per tile
  static constexpr int K_PER_T = (K_UNITS + NT - 1) / NT;
  static constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
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

__device__ inline float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Pack bf16 number `e` (0..7) of four 8-element rows into 4 consecutive bf16 (8 bytes).
__device__ inline u32x2 pick4(const u32x4 (&r)[4], int e) {
  const int w = e >> 1;
  u32x2 out;
  if (e & 1) {
    out[0] = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
    out[1] = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
  } else {
    out[0] = (r[0][w] & 0xffffu) | (r[1][w] << 16);
    out[1] = (r[2][w] & 0xffffu) | (r[3][w] << 16);
  }
  return out;
}

template <int D, class Out>
__global__ __launch_bounds__(NT, 2) void attn_bf16_kernel(const AttnArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int nbh = a.B * a.H;
  const int n_qt = (a.Sq + BM - 1) / BM;
  const int bh = blockIdx.x % nbh;
  const int qt = n_qt - 1 - (int)(blockIdx.x / nbh);  // heaviest (latest) query tile first
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int q0 = qt * BM;
  const int w0 = q0 + wave * 32;
  const int qrow = w0 + l32;
  const bool qvalid = qrow < a.Sq;
  const bool wave_live = w0 < a.Sq;
  const int64_t rs = (int64_t)a.H * D;  // elements between consecutive sequence rows
  const float sl2 = a.scale * kLog2e;

  // ---- Q rows of this wave as B operands (k = head dim), resident for the whole kernel.
  bf16x8 qreg[D / 16];
  {
    const __bf16* qp = (const __bf16*)a.q + ((int64_t)b * a.Sq + qrow) * rs + (int64_t)h * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      if (qvalid) {
        qreg[ks] = *(const bf16x8*)(qp + ks * 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[ks][e] = (__bf16)0.0f;
      }
    }
  }

  // ---- positions of the workgroup's, the wave's and this lane's query rows.
  int64_t wg_qmin = 0, wg_qmax = 0, w_qmin = 0, w_qmax = 0, my_qpos = -1;
  if (a.causal) {
    const int last = min(q0 + BM, a.Sq) - 1;
    wg_qmin = pos_of(a.qpos, q0);
    wg_qmax = pos_of(a.qpos, last);
    if (wave_live) {
      w_qmin = pos_of(a.qpos, w0);
      w_qmax = pos_of(a.qpos, min(w0 + 32, a.Sq) - 1);
    }
    if (qvalid) my_qpos = pos_of(a.qpos, qrow);
  }

  // ---- running state: m (log2 domain), l (this lane half's keys), O^T accumulators.
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

  const int64_t state_row = ((int64_t)b * a.H + h) * a.Sq + qrow;          // [B, H, S]
  const int64_t out_row = (((int64_t)b * a.Sq + qrow) * a.H + h) * D;       // [B, S, H, D]
  if (a.load_state && qvalid) {
    m_run = (float)a.ws_m[state_row];  // stored from this kernel's own fp32 values: exact
    l_run = hh == 0 ? (float)a.ws_l[state_row] : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = *(const f32x4*)(a.ws_o + out_row + db * 32 + g * 8 + hh * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[db][g * 4 + e] = x[e];
      }
  }

  // ---- the (step, tile) sequence this workgroup visits.
  auto share_rule = [&](int s) { return make_pos(a.kv_assign, a.kv_world, a.kv_rank[s], a.kv_len); };
  auto tiles_of = [&](int s) -> int {
    if (!a.causal) return (a.Sk + BN - 1) / BN;
    const int64_t n = clamp64(count_le(share_rule(s), wg_qmax), 0, a.Sk);
    return (int)((n + BN - 1) / BN);
  };

  int s = 0, t = 0;
  int nts = a.nsteps > 0 ? tiles_of(0) : 0;
  bool have = a.nsteps > 0;
  while (have && nts == 0) {
    if (++s >= a.nsteps) { have = false; break; }
    nts = tiles_of(s);
  }

  u32x4 pk[C::K_PER_T];
  u32x4 pv[C::V_PER_T][4];

  auto fetch = [&](int fs, int ft) {
    const __bf16* kb = (const __bf16*)a.k[fs] + (int64_t)b * a.Sk * rs + (int64_t)h * D;
    const __bf16* vb = (const __bf16*)a.v[fs] + (int64_t)b * a.Sk * rs + (int64_t)h * D;
    const int key0 = ft * BN;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int u = tid + i * NT;
      const int key = key0 + u / C::KCH;
      const int ch = u % C::KCH;
      pk[i] = (u32x4){0u, 0u, 0u, 0u};
      if (u < C::K_UNITS && key < a.Sk) pk[i] = *(const u32x4*)(kb + key * rs + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int u = tid + i * NT;
      const int g = u / C::KCH;
      const int ch = u % C::KCH;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = key0 + g * 4 + e;
        pv[i][e] = (u32x4){0u, 0u, 0u, 0u};
        if (u < C::V_UNITS && key < a.Sk) pv[i][e] = *(const u32x4*)(vb + key * rs + ch * 8);
      }
    }
  };

  auto stash = [&](int stage) {
    __bf16* ks_ = smem + stage * C::STAGE;
    __bf16* vt_ = ks_ + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int u = tid + i * NT;
      if (u < C::K_UNITS) *(u32x4*)(ks_ + (u / C::KCH) * C::KS + (u % C::KCH) * 8) = pk[i];
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int u = tid + i * NT;
      if (u < C::V_UNITS) {
        const int g = u / C::KCH;  // keys 4g .. 4g+3 of the tile
        const int ch = u % C::KCH;
        // key index bits: [.. g/4 | bit3 bit2 | bit1 bit0]; stored with bits 2,3 swapped.
        const int col = (g >> 2) * 16 + 4 * (((g & 1) << 1) | ((g >> 1) & 1));
#pragma unroll
        for (int e = 0; e < 8; ++e) *(u32x2*)(vt_ + (ch * 8 + e) * C::VS + col) = pick4(pv[i], e);
      }
    }
  };

  if (have) {
    fetch(s, t);
    stash(0);
  }
  __syncthreads();

  int stage = 0;
  while (have) {
    // next (step, tile)
    int ns = s, nt = t + 1, nnts = nts;
    bool nhave = true;
    while (nt >= nnts) {
      if (++ns >= a.nsteps) { nhave = false; break; }
      nt = 0;
      nnts = tiles_of(ns);
    }
    if (nhave) fetch(ns, nt);

    // classify this tile for the wave
    const Pos kvp = share_rule(s);
    const int key0 = t * BN;
    const int klast = min(key0 + BN, a.Sk) - 1;
    bool skip = !wave_live;
    bool masked = key0 + BN > a.Sk;
    if (a.causal && wave_live) {
      const int64_t kmin = pos_of(kvp, key0);
      const int64_t kmax = pos_of(kvp, klast);
      skip = w_qmax < kmin;
      masked = masked || (w_qmin < kmax);
    }

    if (!skip) {
      const __bf16* ks_ = smem + stage * C::STAGE;
      const __bf16* vt_ = ks_ + C::K_ELEMS;
      f32x16 sacc[BN / 32];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 ka = *(const bf16x8*)(ks_ + (kb * 32 + l32) * C::KS + ks * 16 + hh * 8);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], sacc[kb], 0, 0, 0);
        }
      }
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
            bool vis = key < a.Sk;
            if (a.causal) vis = vis && visible(my_qpos, pos_of(kvp, key));
            if (!vis) sacc[kb][r] = -INFINITY;
          }
      }
      // online softmax update (log2 domain)
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = fmaxf(mt, xor32(mt));
      const float m_new = fmaxf(m_run, mt * sl2);
      const float base = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - base);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

      bf16x8 pb[BN / 32][2];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], sl2, -base));
          l_run += p;
          pb[kb][r >> 3][r & 7] = (__bf16)p;
        }
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const bf16x8 va = *(const bf16x8*)(vt_ + (db * 32 + l32) * C::VS + kb * 32 + j * 16 + hh * 8);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][j], oacc[db], 0, 0, 0);
          }
    }

    if (nhave) stash(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    s = ns;
    t = nt;
    nts = nnts;
    have = nhave;
  }

  // ---- epilogue
  const float l_tot = l_run + xor32(l_run);
  if (!qvalid) return;
  if (a.store_final) {
    const bool any = l_tot > 0.f;
    const float inv = any ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = oacc[db][g * 4 + e] * inv;
        Out::store4(a.o, out_row + db * 32 + g * 8 + hh * 4, x);
      }
    if (hh == 0) a.lse[state_row] = any ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  } else {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = oacc[db][g * 4 + e];
        *(f32x4*)(a.ws_o + out_row + db * 32 + g * 8 + hh * 4) = x;
      }
    if (hh == 0) {
      a.ws_m[state_row] = m_run;
      a.ws_l[state_row] = l_tot;
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, int D, int o_dtype, hipStream_t stream) {
  const int n_qt = (a.Sq + BM - 1) / BM;
  const int64_t grid = (int64_t)n_qt * a.B * a.H;
  if (grid == 0) return hipSuccess;
  dim3 g((unsigned)grid), blk(NT);
  if (D == 128) {
    if (o_dtype == RA_BF16) hipLaunchKernelGGL((attn_bf16_kernel<128, OutBf16>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<128, OutF32>), g, blk, 0, stream, a);
  } else {
    if (o_dtype == RA_BF16) hipLaunchKernelGGL((attn_bf16_kernel<64, OutBf16>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<64, OutF32>), g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ra
