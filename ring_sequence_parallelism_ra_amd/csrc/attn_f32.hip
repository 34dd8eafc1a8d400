// Blockwise attention with the online-softmax update for fp32 inputs (fp32 FMA, no MFMA).
//
// Same computation as the bf16 kernel ([Digest] = "从 Ring Attention 到 DeepSpeed Ulysses，
// 再到 USP 统一框架": definition §2, ring order §3.1/§3.3, update §3.2, causal matrix §3.4)
// for the small fp32 checks, where accuracy matters and speed does not. One lane owns one
// query row; a wave64 workgroup owns 64 rows of one (batch, head). K/V tiles of 32 keys
// are staged in LDS and read by every lane as broadcasts. Logits, the running max and sum and
// the LSE are carried in fp64 (exact products of the fp32 inputs, device-library exp/log in
// double), so the only fp32 rounding of the LSE is the final store; O accumulates in fp32.
#include <math.h>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int BM = kF32BlockM;  // query rows per workgroup (one per lane)
constexpr int BN = kF32BlockN;  // keys per tile

template <int D, typename OutT>
__global__ __launch_bounds__(BM) void attn_f32_kernel(const AttnArgs a) {
  __shared__ float ks_[BN * D];
  __shared__ float vs_[BN * D];
  __shared__ float qs_[BM * (D + 1)];  // this lane's query row, padded against bank conflicts

  const int lane = threadIdx.x;
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
  for (int d = 0; d < D; ++d) q[d] = qvalid ? qp[d] : 0.f;

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
  if (a.load_state && qvalid) {
    m_run = a.ws_m[state_row];
    l_run = a.ws_l[state_row];  // fp64 state slots
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = a.ws_o[out_row + d];
  }

  for (int s = 0; s < a.nsteps; ++s) {
    const Pos kvp = make_pos(a.kv_assign, a.kv_world, a.kv_rank[s], a.kv_len);
    int32_t nvis = a.Sk;
    if (a.causal) nvis = clamp32(count_le(kvp, wg_qmax), 0, a.Sk);
    const float* kb = (const float*)a.k[s] + (int64_t)b * a.Sk * rs_kv + (int64_t)hk * D;
    const float* vb = (const float*)a.v[s] + (int64_t)b * a.Sk * rs_kv + (int64_t)hk * D;
    for (int key0 = 0; key0 < nvis; key0 += BN) {
      __syncthreads();
      for (int u = lane; u < BN * D; u += BM) {
        const int j = u / D, d = u % D;
        const int key = key0 + j;
        ks_[u] = key < a.Sk ? kb[key * rs_kv + d] : 0.f;
        vs_[u] = key < a.Sk ? vb[key * rs_kv + d] : 0.f;
      }
      __syncthreads();
      double sc[BN];
      double mt = -INFINITY;
      for (int j = 0; j < BN; ++j) {
        double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, acc3 = 0.0;
#pragma unroll 8
        for (int d = 0; d < D; d += 4) {
          acc0 = fma((double)q[d + 0], (double)ks_[j * D + d + 0], acc0);
          acc1 = fma((double)q[d + 1], (double)ks_[j * D + d + 1], acc1);
          acc2 = fma((double)q[d + 2], (double)ks_[j * D + d + 2], acc2);
          acc3 = fma((double)q[d + 3], (double)ks_[j * D + d + 3], acc3);
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
      for (int j = 0; j < BN; ++j) {
        const double p = exp(sc[j] - base);
        l_run += p;
        const float pf = (float)p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(pf, vs_[j * D + d], o[d]);
      }
    }
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

hipError_t launch_attn_f32(const AttnArgs& a, int D, int o_dtype, hipStream_t stream) {
  const int n_qt = (a.Sq + BM - 1) / BM;
  const int64_t grid = (int64_t)n_qt * a.B * a.H;
  if (grid == 0) return hipSuccess;
  dim3 g((unsigned)grid), blk(BM);
  if (D == 128) {
    if (o_dtype == RA_BF16) hipLaunchKernelGGL((attn_f32_kernel<128, __bf16>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((attn_f32_kernel<128, float>), g, blk, 0, stream, a);
  } else {
    if (o_dtype == RA_BF16) hipLaunchKernelGGL((attn_f32_kernel<64, __bf16>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((attn_f32_kernel<64, float>), g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ra
