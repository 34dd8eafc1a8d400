// Blockwise attention with the online-softmax update for fp32 inputs (fp32 FMA, no MFMA).
//
// Same computation as the bf16 kernel ([Digest] = "从 Ring Attention 到 DeepSpeed Ulysses，
// 再到 USP 统一框架": definition §2, ring order §3.1/§3.3, update §3.2, causal matrix §3.4)
// for the small fp32 checks, where accuracy matters and speed does not. One lane owns one
// query row; a wave64 workgroup owns 64 rows of one (batch, head). K/V tiles of 32 keys
// are staged in LDS and read by every lane as broadcasts. Logits, the running max and sum and
// the LSE are carried in fp64 (exact products of the fp32 inputs, device-library exp/log in
// double), so the only fp32 rounding of the LSE is the final store; O accumulates in fp32.
// Small grids (fewer workgroups than CUs, e.g. one 64-query share) use NW = 4 waves on the same
// 64 rows: wave w folds every NW-th key tile (16 keys) into its own state, and the states are
// merged at the end with the log-sum-exp update (fp64 maximum and sum).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int BM = kF32BlockM;  // query rows per workgroup (one per lane)
constexpr int BN = kF32BlockN;  // keys per tile

template <int D, typename OutT, int NW>
__global__ __launch_bounds__(BM * NW) void attn_f32_kernel(const AttnArgs a) {
  constexpr int TBN = NW == 1 ? BN : 16;  // keys per tile
  __shared__ float ks_[NW * TBN * D];
  __shared__ float vs_[NW * TBN * D];
  __shared__ float qs_[BM * (D + 1)];  // this lane's query row, padded against bank conflicts
  static_assert(NW == 1 || NW * TBN * D >= BM * D, "the merge stages a wave's O in ks_");

  const int lane = threadIdx.x % BM;
  const int w = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / BM);
  float* kt_ = ks_ + w * TBN * D;  // this wave's tile buffers
  float* vt_ = vs_ + w * TBN * D;
  const int nbh = a.B * a.H;
  const int n_qt = (a.Sq + BM - 1) / BM;
  const int bh = blockIdx.x % nbh;
  const int qt = n_qt - 1 - (int)(blockIdx.x / nbh);
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int q0 = qt * BM;
  const int qrow = q0 + lane;
  const bool qvalid = qrow < a.Sq;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t rs_kv = (int64_t)a.Hkv * D;  // K/V rows hold Hkv heads; query head h reads h / (H / Hkv)
  const int hk = h / (a.H / a.Hkv);

  const float* qp = (const float*)a.q + ((int64_t)b * a.Sq + qrow) * rs + (int64_t)h * D;
  float* q = qs_ + lane * (D + 1);
  if (w == 0)
    for (int d = 0; d < D; ++d) q[d] = qvalid ? qp[d] : 0.f;
  if constexpr (NW > 1) __syncthreads();

  int32_t wg_qmax = 0, my_qpos = -1;
  if (a.causal) {
    wg_qmax = pos_of(a.qpos, min(q0 + BM, a.Sq) - 1);
    if (qvalid) my_qpos = pos_of(a.qpos, qrow);
  }

  double m_run = -INFINITY, l_run = 0.0;
  const double scale = a.scale;
  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  const int64_t state_row = ((int64_t)b * a.H + h) * a.Sq + qrow;
  const int64_t out_row = (((int64_t)b * a.Sq + qrow) * a.H + h) * D;
  if (a.load_state && qvalid && w == 0) {
    m_run = a.ws_m[state_row];
    l_run = a.ws_l[state_row];  // fp64 state slots
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = a.ws_o[out_row + d];
  }

  int tile_no = 0;  // tiles of the call so far (wave w takes those with tile_no % NW == w)
  for (int s = 0; s < a.nsteps; ++s) {
    const Pos kvp = make_pos(a.kv_assign, a.kv_world, a.kv_rank[s], a.kv_len);
    int32_t nvis = a.Sk;
    if (a.causal) nvis = clamp32(count_le(kvp, wg_qmax), 0, a.Sk);
    const float* kb = (const float*)a.k[s] + (int64_t)b * a.Sk * rs_kv + (int64_t)hk * D;
    const float* vb = (const float*)a.v[s] + (int64_t)b * a.Sk * rs_kv + (int64_t)hk * D;
    for (int key0 = 0; key0 < nvis; key0 += TBN) {
      if constexpr (NW > 1) {
        if (tile_no++ % NW != w) continue;
      }
      // the wave's previous reads of its tile buffers are done before they are overwritten
      if constexpr (NW == 1) __syncthreads();
      else __builtin_amdgcn_s_waitcnt(0), __builtin_amdgcn_wave_barrier();
      for (int u = lane; u < TBN * D; u += BM) {
        const int j = u / D, d = u % D;
        const int key = key0 + j;
        kt_[u] = key < a.Sk ? kb[key * rs_kv + d] : 0.f;
        vt_[u] = key < a.Sk ? vb[key * rs_kv + d] : 0.f;
      }
      if constexpr (NW == 1) __syncthreads();
      else __builtin_amdgcn_s_waitcnt(0), __builtin_amdgcn_wave_barrier();
      double sc[TBN];
      double mt = -INFINITY;
      for (int j = 0; j < TBN; ++j) {
        double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, acc3 = 0.0;
#pragma unroll 8
        for (int d = 0; d < D; d += 4) {
          acc0 = fma((double)q[d + 0], (double)kt_[j * D + d + 0], acc0);
          acc1 = fma((double)q[d + 1], (double)kt_[j * D + d + 1], acc1);
          acc2 = fma((double)q[d + 2], (double)kt_[j * D + d + 2], acc2);
          acc3 = fma((double)q[d + 3], (double)kt_[j * D + d + 3], acc3);
        }
        double sj = ((acc0 + acc1) + (acc2 + acc3)) * scale;
        const int key = key0 + j;
        bool vis = key < a.Sk;
        if (a.causal) vis = vis && visible(my_qpos, pos_of(kvp, key));
        sj = vis ? sj : -INFINITY;
        sc[j] = sj;
        mt = fmax(mt, sj);
      }
      const double m_new = fmax(m_run, mt);
      const double base = m_new == -INFINITY ? 0.0 : m_new;
      const double alpha = exp(m_run - base);
      m_run = m_new;
      l_run *= alpha;
      const float alpha_f = (float)alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha_f;
      for (int j = 0; j < TBN; ++j) {
        const double p = exp(sc[j] - base);
        l_run += p;
        const float pf = (float)p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(pf, vt_[j * D + d], o[d]);
      }
    }
  }

  if constexpr (NW > 1) {
    // Merge wave k's state into wave 0's, one wave at a time: O staged lane-contiguously in ks_,
    // (m, l) in vs_ as doubles; a side that has seen no key contributes nothing.
    double* ml = (double*)vs_;
    for (int k = 1; k < NW; ++k) {
      __syncthreads();  // every wave is done with its tiles (k = 1) / wave 0 with the last merge
      if (w == k) {
#pragma unroll
        for (int d = 0; d < D; ++d) ks_[d * BM + lane] = o[d];
        ml[lane] = m_run;
        ml[BM + lane] = l_run;
      }
      __syncthreads();
      if (w == 0) {
        const double mk = ml[lane], lk = ml[BM + lane];
        const double m = fmax(m_run, mk);
        const double f0 = m_run == -INFINITY ? 0.0 : exp(m_run - m);
        const double fk = mk == -INFINITY ? 0.0 : exp(mk - m);
        m_run = m;
        l_run = l_run * f0 + lk * fk;
        const float f0f = (float)f0, fkf = (float)fk;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = o[d] * f0f + ks_[d * BM + lane] * fkf;
      }
    }
    if (w != 0) return;
  }

  if (!qvalid) return;
  if (a.store_final) {
    const bool any = l_run > 0.0;
    const double inv = any ? 1.0 / l_run : 0.0;
    OutT* op = (OutT*)a.o + out_row;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = (OutT)(float)(o[d] * inv);
    a.lse[state_row] = any ? (float)(m_run + log(l_run)) : -INFINITY;
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) a.ws_o[out_row + d] = o[d];
    a.ws_m[state_row] = m_run;
    a.ws_l[state_row] = l_run;
  }
}

}  // namespace

template <int NW>
static void launch_f32(const AttnArgs& a, int D, int o_dtype, dim3 g, hipStream_t stream) {
  dim3 blk(BM * NW);
  if (D == 128) {
    if (o_dtype == RA_BF16) hipLaunchKernelGGL((attn_f32_kernel<128, __bf16, NW>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((attn_f32_kernel<128, float, NW>), g, blk, 0, stream, a);
  } else {
    if (o_dtype == RA_BF16) hipLaunchKernelGGL((attn_f32_kernel<64, __bf16, NW>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((attn_f32_kernel<64, float, NW>), g, blk, 0, stream, a);
  }
}

hipError_t launch_attn_f32(const AttnArgs& a, int D, int o_dtype, hipStream_t stream) {
  const int n_qt = (a.Sq + BM - 1) / BM;
  const int64_t grid = (int64_t)n_qt * a.B * a.H;
  if (grid == 0) return hipSuccess;
  // Key split (four waves per 64-row query tile) for grids that leave most CUs idle; the same
  // RA_KV_SPLIT override as the bf16 kernel ("always" / "never").
  const char* e = getenv("RA_KV_SPLIT");
  const int mode = !e ? 0 : !strcmp(e, "always") ? 1 : !strcmp(e, "never") ? -1 : 0;
  if (mode > 0 || (mode == 0 && grid < 256)) launch_f32<4>(a, D, o_dtype, dim3((unsigned)grid), stream);
  else launch_f32<1>(a, D, o_dtype, dim3((unsigned)grid), stream);
  return hipGetLastError();
}

}  // namespace ra
