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
// One launch moves up to kMaxPermute tensors of the same shape (blockIdx.y picks the tensor),
// so the Q, K and V of a Ulysses step go in one grid. IDX is the index type: 32-bit when every
// offset of a tensor fits (cheap division), 64-bit otherwise.
template <int VEC>
struct VecT;
template <>
struct VecT<16> { typedef u32x4 type; };
template <>
struct VecT<4> { typedef uint32_t type; };
template <>
struct VecT<2> { typedef uint16_t type; };

struct PermuteArgs {
  const char* in[kMaxPermute];
  char* out[kMaxPermute];
};

template <int VEC, typename IDX>
__global__ __launch_bounds__(256) void permute_kernel(const PermuteArgs t, IDX B, IDX P, IDX S,
                                                      IDX row_bytes, IDX in_row_bytes, IDX first_rank,
                                                      IDX n_ranks, int inverse) {
  typedef typename VecT<VEC>::type vec_t;
  const char* __restrict__ in = t.in[blockIdx.y];
  char* __restrict__ out = t.out[blockIdx.y];
  const IDX per_row = row_bytes / VEC;
  const IDX rows = P * B * S;
  const IDX n = per_row * rows * n_ranks;
  const IDX stride = (IDX)gridDim.x * blockDim.x;
  for (IDX u = (IDX)blockIdx.x * blockDim.x + threadIdx.x; u < n; u += stride) {
    const IDX r = u / per_row;
    const IDX c = u - r * per_row;
    const IDX k = r / rows;            // which destination rank of the batch
    const IDX row = r - k * rows;      // index over (b, src, s) in head-sharded order
    const IDX bsrc = row / S;
    const IDX s = row - bsrc * S;
    const IDX b = bsrc / P;
    const IDX src = bsrc - b * P;
    const IDX dst = first_rank + k;
    // sequence-sharded side: [P, B, S, H*D], slice of rank dst
    const IDX seq_off = ((src * B + b) * S + s) * in_row_bytes + dst * row_bytes + c * VEC;
    // head-sharded side: [n_ranks, B, P*S, Hp*D] (consecutive u: consecutive bytes)
    const IDX head_off = r * row_bytes + c * VEC;
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

template <int VEC, typename IDX>
static void launch_permute_t(const PermuteArgs& t, int n_t, int64_t B, int64_t P, int64_t S_loc, int64_t row_bytes,
                             int64_t in_row_bytes, int64_t first, int64_t nr, int inverse, hipStream_t stream) {
  const int64_t n = row_bytes * P * B * S_loc * nr / VEC;
  const int64_t blocks = (n + 255) / 256;
  const dim3 blk(256), g((unsigned)(blocks < 1048576 ? blocks : 1048576), (unsigned)n_t);
  hipLaunchKernelGGL((permute_kernel<VEC, IDX>), g, blk, 0, stream, t, (IDX)B, (IDX)P, (IDX)S_loc, (IDX)row_bytes,
                     (IDX)in_row_bytes, (IDX)first, (IDX)nr, inverse);
}

template <typename IDX>
static void launch_permute_v(int vec, const PermuteArgs& t, int n_t, int64_t B, int64_t P, int64_t S_loc,
                             int64_t row_bytes, int64_t in_row_bytes, int64_t first, int64_t nr, int inverse,
                             hipStream_t stream) {
  if (vec == 16) launch_permute_t<16, IDX>(t, n_t, B, P, S_loc, row_bytes, in_row_bytes, first, nr, inverse, stream);
  else if (vec == 4) launch_permute_t<4, IDX>(t, n_t, B, P, S_loc, row_bytes, in_row_bytes, first, nr, inverse, stream);
  else launch_permute_t<2, IDX>(t, n_t, B, P, S_loc, row_bytes, in_row_bytes, first, nr, inverse, stream);
}

hipError_t launch_permute(const void* const* in, void* const* out, int n_t, int64_t B, int64_t P, int64_t S_loc,
                          int64_t H, int64_t D, int esize, int dst_rank, int inverse, hipStream_t stream) {
  const int64_t hp = H / P;
  const int64_t row_bytes = hp * D * esize;
  const int64_t in_row_bytes = H * D * esize;
  const int64_t first = dst_rank < 0 ? 0 : dst_rank;
  const int64_t nr = dst_rank < 0 ? P : 1;
  const int64_t total = row_bytes * P * B * S_loc * nr;
  if (total == 0 || n_t == 0) return hipSuccess;
  PermuteArgs t;
  uintptr_t any = 0;
  for (int i = 0; i < kMaxPermute; ++i) {
    t.in[i] = i < n_t ? (const char*)in[i] : nullptr;
    t.out[i] = i < n_t ? (char*)out[i] : nullptr;
    if (i < n_t) any |= (uintptr_t)in[i] | (uintptr_t)out[i];
  }
  const bool v16 = row_bytes % 16 == 0 && any % 16 == 0;
  const int vec = v16 ? 16 : (row_bytes % 4 == 0 ? 4 : 2);
  // every byte offset of one tensor (both sides span P*B*S_loc*H*D elements) below 2^31
  const bool small = P * B * S_loc * H * D * esize < ((int64_t)1 << 31);
  if (small) launch_permute_v<uint32_t>(vec, t, n_t, B, P, S_loc, row_bytes, in_row_bytes, first, nr, inverse, stream);
  else launch_permute_v<uint64_t>(vec, t, n_t, B, P, S_loc, row_bytes, in_row_bytes, first, nr, inverse, stream);
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
