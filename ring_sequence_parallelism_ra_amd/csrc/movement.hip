// HBM-bound kernels: the LSE merge, the Ulysses sequence<->head permute, and the debug
// hooks that expose the position rule and the causal mask.
//
// [Digest] = "从 Ring Attention 到 DeepSpeed Ulysses，再到 USP 统一框架" (jsqmd.com):
//   merge   -- "merge_lse" of §6 item 3: lse = max(a,b) + log(1 + e^{-|a-b|}),
//              O = O_a e^{a-lse} + O_b e^{b-lse} (normalised O's, nothing further divided);
//   permute -- the layout change around the Ulysses all-to-all of §5.1: rank p gets the whole
//              sequence (ordered by source rank) for heads [p*H/P, (p+1)*H/P).
// Both are streaming kernels: every thread moves 16 bytes per access with 128-bit loads and
// stores, consecutive threads touch consecutive addresses.
#include <math.h>

#include "ra_internal.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec8;
template <>
struct Vec8<float> {
  static __device__ inline void load(const void* p, int64_t off, float (&x)[8]) {
    const f32x4 a = *(const f32x4*)((const float*)p + off);
    const f32x4 b = *(const f32x4*)((const float*)p + off + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[i + 4] = b[i];
    }
  }
  static __device__ inline void store(void* p, int64_t off, const float (&x)[8]) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = x[i];
      b[i] = x[i + 4];
    }
    *(f32x4*)((float*)p + off) = a;
    *(f32x4*)((float*)p + off + 4) = b;
  }
};
template <>
struct Vec8<__bf16> {
  static __device__ inline void load(const void* p, int64_t off, float (&x)[8]) {
    const bf16x8 a = *(const bf16x8*)((const __bf16*)p + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)a[i];
  }
  static __device__ inline void store(void* p, int64_t off, const float (&x)[8]) {
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (__bf16)x[i];
    *(bf16x8*)((__bf16*)p + off) = a;
  }
};

// One thread per 8 consecutive elements of one (b, s, h) row of O.
template <typename TA, typename TB>
__global__ __launch_bounds__(256) void lse_merge_kernel(void* __restrict__ o_acc, float* __restrict__ lse_acc,
                                                        const void* __restrict__ o_blk,
                                                        const float* __restrict__ lse_blk, int64_t S,
                                                        int64_t H, int64_t D, int64_t n_units) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= n_units) return;
  const int64_t per_row = D / 8;
  const int64_t row = u / per_row;  // (b, s, h) row of O
  const int64_t chunk = u % per_row;
  const int64_t h = row % H;
  const int64_t s = (row / H) % S;
  const int64_t b = row / (H * S);
  const int64_t li = (b * H + h) * S + s;
  // The LSE arithmetic runs in fp64 on the fp32 inputs so that the merged LSE is rounded
  // once, at the store.
  const double la = lse_acc[li];
  const double lb = lse_blk[li];
  const bool fa = la != -INFINITY, fb = lb != -INFINITY;
  double lse;
  float wa, wb;
  if (fa && fb) {
    const double hi = fmax(la, lb);
    lse = hi + log1p(exp(-fabs(la - lb)));
    wa = (float)exp(la - lse);
    wb = (float)exp(lb - lse);
  } else if (fa) {
    lse = la, wa = 1.f, wb = 0.f;
  } else if (fb) {
    lse = lb, wa = 0.f, wb = 1.f;
  } else {
    lse = -INFINITY, wa = 0.f, wb = 0.f;
  }
  const int64_t off = row * D + chunk * 8;
  float xa[8], xb[8];
  Vec8<TA>::load(o_acc, off, xa);
  Vec8<TB>::load(o_blk, off, xb);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (wa == 0.f ? 0.f : xa[i] * wa) + (wb == 0.f ? 0.f : xb[i] * wb);
  Vec8<TA>::store(o_acc, off, y);
  if (chunk == 0) lse_acc[li] = (float)lse;
}

// Sequence-sharded [P, B, S, H, D] <-> head-sharded [B, P*S, H/P, D] (per destination rank).
// A "row" is one (src, b, s) position: its destination-rank slice is Hp*D contiguous
// elements on both sides. VEC = bytes moved per access (16 when rows and offsets allow).
template <int VEC>
struct VecT;
template <>
struct VecT<16> { typedef u32x4 type; };
template <>
struct VecT<4> { typedef uint32_t type; };
template <>
struct VecT<2> { typedef uint16_t type; };

template <int VEC>
__global__ __launch_bounds__(256) void permute_kernel(const char* __restrict__ in, char* __restrict__ out,
                                                      int64_t B, int64_t P, int64_t S, int64_t H,
                                                      int64_t row_bytes, int64_t in_row_bytes,
                                                      int64_t first_rank, int64_t n_ranks, int inverse) {
  typedef typename VecT<VEC>::type vec_t;
  const int64_t per_row = row_bytes / VEC;
  const int64_t rows = P * B * S;
  const int64_t n = per_row * rows * n_ranks;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = u % per_row;
    const int64_t r = u / per_row;
    const int64_t row = r % rows;      // index over (b, src, s) in head-sharded order
    const int64_t k = r / rows;        // which destination rank of the batch
    const int64_t dst = first_rank + k;
    const int64_t s = row % S;
    const int64_t src = (row / S) % P;
    const int64_t b = row / (S * P);
    // sequence-sharded side: [P, B, S, H*D], slice of rank dst
    const int64_t seq_off = ((src * B + b) * S + s) * in_row_bytes + dst * row_bytes + c * VEC;
    // head-sharded side: [n_ranks, B, P*S, Hp*D]
    const int64_t head_off = ((k * B + b) * (P * S) + src * S + s) * row_bytes + c * VEC;
    if (!inverse) {
      *(vec_t*)(out + head_off) = *(const vec_t*)(in + seq_off);
    } else {
      *(vec_t*)(out + seq_off) = *(const vec_t*)(in + head_off);
    }
  }
}

__global__ void positions_kernel(Pos p, int64_t n, int64_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = pos_of(p, (int32_t)i);
}

__global__ void mask_kernel(Pos q, Pos kv, int64_t Sq, int64_t Sk, uint8_t* out) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= Sq * Sk) return;
  const int64_t i = u / Sk, j = u % Sk;
  out[u] = visible(pos_of(q, (int32_t)i), pos_of(kv, (int32_t)j)) ? 1 : 0;
}

}  // namespace

hipError_t launch_lse_merge(void* o_acc, float* lse_acc, const void* o_blk, const float* lse_blk,
                            int64_t B, int64_t H, int64_t S, int64_t D, int acc_dtype,
                            int blk_dtype, hipStream_t stream) {
  const int64_t n_units = B * S * H * (D / 8);
  if (n_units == 0) return hipSuccess;
  const dim3 blk(256), g((unsigned)((n_units + 255) / 256));
  if (acc_dtype == RA_F32 && blk_dtype == RA_F32)
    hipLaunchKernelGGL((lse_merge_kernel<float, float>), g, blk, 0, stream, o_acc, lse_acc, o_blk, lse_blk, S, H, D, n_units);
  else if (acc_dtype == RA_F32)
    hipLaunchKernelGGL((lse_merge_kernel<float, __bf16>), g, blk, 0, stream, o_acc, lse_acc, o_blk, lse_blk, S, H, D, n_units);
  else if (blk_dtype == RA_F32)
    hipLaunchKernelGGL((lse_merge_kernel<__bf16, float>), g, blk, 0, stream, o_acc, lse_acc, o_blk, lse_blk, S, H, D, n_units);
  else
    hipLaunchKernelGGL((lse_merge_kernel<__bf16, __bf16>), g, blk, 0, stream, o_acc, lse_acc, o_blk, lse_blk, S, H, D, n_units);
  return hipGetLastError();
}

hipError_t launch_permute(const void* in, void* out, int64_t B, int64_t P, int64_t S_loc,
                          int64_t H, int64_t D, int esize, int dst_rank, int inverse,
                          hipStream_t stream) {
  const int64_t hp = H / P;
  const int64_t row_bytes = hp * D * esize;
  const int64_t in_row_bytes = H * D * esize;
  const int64_t first = dst_rank < 0 ? 0 : dst_rank;
  const int64_t nr = dst_rank < 0 ? P : 1;
  const int64_t total = row_bytes * P * B * S_loc * nr;
  if (total == 0) return hipSuccess;
  const bool v16 = row_bytes % 16 == 0 && (((uintptr_t)in | (uintptr_t)out) % 16) == 0;
  const int vec = v16 ? 16 : (row_bytes % 4 == 0 ? 4 : 2);
  const int64_t n = total / vec;
  const int64_t blocks = (n + 255) / 256;
  const dim3 blk(256), g((unsigned)(blocks < 1048576 ? blocks : 1048576));
  if (vec == 16)
    hipLaunchKernelGGL((permute_kernel<16>), g, blk, 0, stream, (const char*)in, (char*)out, B, P, S_loc, H, row_bytes, in_row_bytes, first, nr, inverse);
  else if (vec == 4)
    hipLaunchKernelGGL((permute_kernel<4>), g, blk, 0, stream, (const char*)in, (char*)out, B, P, S_loc, H, row_bytes, in_row_bytes, first, nr, inverse);
  else
    hipLaunchKernelGGL((permute_kernel<2>), g, blk, 0, stream, (const char*)in, (char*)out, B, P, S_loc, H, row_bytes, in_row_bytes, first, nr, inverse);
  return hipGetLastError();
}

hipError_t launch_debug_positions(Pos p, int64_t n, int64_t* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(positions_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n, out);
  return hipGetLastError();
}

hipError_t launch_debug_mask(Pos q, Pos kv, int64_t Sq, int64_t Sk, uint8_t* out, hipStream_t stream) {
  const int64_t n = Sq * Sk;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mask_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, q, kv, Sq, Sk, out);
  return hipGetLastError();
}

}  // namespace ra
