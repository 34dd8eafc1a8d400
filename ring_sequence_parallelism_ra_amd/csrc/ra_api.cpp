// Host side of the C ABI declared in include/ra.h: argument validation (all of it before any
// launch, so every error path runs without a GPU), the ring step order, workspace layout,
// the planner counts and the kernel launches.
//
// [Digest] = "从 Ring Attention 到 DeepSpeed Ulysses，再到 USP 统一框架" (jsqmd.com).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <unordered_map>

#include "ra_internal.h"

namespace {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return RA_OK;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

bool dtype_ok(int d) { return d == RA_F32 || d == RA_BF16; }

int check_shard(const ra_shard* sh, int64_t S, const char* what) {
  if (!sh) return fail(RA_ERR_INVALID_ARG, "%s: shard descriptor is NULL", what);
  if (sh->assign < RA_CONTIGUOUS || sh->assign > RA_ZIGZAG)
    return fail(RA_ERR_INVALID_ARG, "%s: unknown assignment %d", what, sh->assign);
  if (sh->world < 1) return fail(RA_ERR_INVALID_ARG, "%s: world %d < 1", what, sh->world);
  if (sh->rank < 0 || sh->rank >= sh->world)
    return fail(RA_ERR_INVALID_ARG, "%s: rank %d not in [0, %d)", what, sh->rank, sh->world);
  if (sh->global_len < 0) return fail(RA_ERR_INVALID_ARG, "%s: negative global_len", what);
  if (sh->global_len >= ((int64_t)1 << 31))
    return fail(RA_ERR_UNSUPPORTED, "%s: global_len %lld >= 2^31", what, (long long)sh->global_len);
  const int64_t parts = sh->assign == RA_ZIGZAG ? 2 * (int64_t)sh->world : sh->world;
  if (sh->global_len % parts)
    return fail(RA_ERR_SHAPE, "%s: global_len %lld not divisible by %lld", what,
                (long long)sh->global_len, (long long)parts);
  if (S >= 0 && sh->global_len / sh->world != S)
    return fail(RA_ERR_SHAPE, "%s: share length %lld != global_len/world = %lld", what, (long long)S,
                (long long)(sh->global_len / sh->world));
  return RA_OK;
}

ra::Pos to_pos(const ra_shard& s) { return ra::make_pos(s.assign, s.world, s.rank, s.global_len); }

// Sizes must fit the kernels' 32-bit row indices.
int check_dims(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D) {
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || D < 0) return fail(RA_ERR_INVALID_ARG, "negative size");
  if (D != 64 && D != 128) return fail(RA_ERR_UNSUPPORTED, "head dim D=%lld not in {64, 128}", (long long)D);
  const int64_t lim = (int64_t)1 << 30;
  if (B * H >= lim || Sq >= lim || Sk >= lim)
    return fail(RA_ERR_UNSUPPORTED, "sizes too large for 32-bit row indexing");
  // byte offsets inside one 64-row K/V tile (rows of H*D elements) are 32-bit, and the bytes of
  // one K/V row are multiplied with 24-bit multiplies when the tiles are copied
  if (H * D * 2 >= ((int64_t)1 << 24))
    return fail(RA_ERR_UNSUPPORTED, "H*D=%lld: rows of 2^24 bytes or more are not supported", (long long)(H * D));
  // one workgroup per (64-row query tile, batch, head) must fit a 32-bit grid
  if ((Sq + 63) / 64 * B * H >= ((int64_t)1 << 31))
    return fail(RA_ERR_UNSUPPORTED, "launch grid too large");
  return RA_OK;
}

// KV heads for grouped-query attention: 1 <= H_kv and H_kv divides H (H_kv = H: plain
// multi-head; 1: multi-query). Ignored when H == 0.
int check_kv_heads(int64_t H, int64_t H_kv) {
  if (H == 0) return H_kv < 0 ? fail(RA_ERR_INVALID_ARG, "negative H_kv") : RA_OK;
  if (H_kv < 1) return fail(RA_ERR_INVALID_ARG, "H_kv=%lld < 1", (long long)H_kv);
  if (H % H_kv)
    return fail(RA_ERR_SHAPE, "H_kv=%lld does not divide H=%lld", (long long)H_kv, (long long)H);
  return RA_OK;
}

// What a resume workspace holds. The running state's layout depends on the kernel that wrote
// it (the bf16 kernel keeps the running max in log2 units of scaled logits, the fp32 kernel in
// natural units), so a state may only be resumed by a call with the same arguments, at the step
// where the storing call stopped. The record is kept on the host, per workspace address, for
// every call that stores a state; a resume is checked against it before anything is launched.
struct WsTag {
  int in_dtype, assign, causal, N, rank;
  int64_t B, H, H_kv, S, D;
  uint32_t scale_bits;
  int next_step;  // the first step the stored state has not folded in
};

std::mutex g_ws_mu;
std::unordered_map<uintptr_t, WsTag>& ws_tags() {
  static std::unordered_map<uintptr_t, WsTag> m;
  return m;
}

// RA_OK if `want` (with next_step = the resuming call's start_step) may resume the state in ws.
int check_resume(const void* ws, const WsTag& want) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto it = ws_tags().find((uintptr_t)ws);
  if (it == ws_tags().end())
    return fail(RA_ERR_INVALID_ARG, "resume: no running state was stored in this workspace by this process");
  const WsTag& t = it->second;
  if (t.in_dtype != want.in_dtype)
    return fail(RA_ERR_INVALID_ARG, "resume: state stored with in_dtype %d, resumed with %d", t.in_dtype, want.in_dtype);
  if (t.scale_bits != want.scale_bits) return fail(RA_ERR_INVALID_ARG, "resume: state stored with another scale");
  if (t.assign != want.assign || t.causal != want.causal || t.N != want.N || t.rank != want.rank)
    return fail(RA_ERR_INVALID_ARG, "resume: state stored for another ring (assignment, mask, N or rank)");
  if (t.B != want.B || t.H != want.H || t.H_kv != want.H_kv || t.S != want.S || t.D != want.D)
    return fail(RA_ERR_INVALID_ARG, "resume: state stored for another shape");
  if (t.next_step != want.next_step)
    return fail(RA_ERR_INVALID_ARG, "resume: state covers steps up to %d, call starts at step %d", t.next_step,
                want.next_step);
  return RA_OK;
}

void record_state(const void* ws, const WsTag& tag) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  ws_tags()[(uintptr_t)ws] = tag;
}

int launch_attn(const ra::AttnArgs& a, int D, int in_dtype, int o_dtype, hipStream_t stream) {
  hipError_t e = in_dtype == RA_BF16 ? ra::launch_attn_bf16(a, D, o_dtype, stream)
                                     : ra::launch_attn_f32(a, D, o_dtype, stream);
  if (e != hipSuccess) return fail(RA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* ra_last_error(void) { return g_err; }

int ra_tile_shape(int in_dtype, int64_t D, int64_t* block_m, int64_t* block_n) {
  if (!block_m || !block_n) return fail(RA_ERR_INVALID_ARG, "ra_tile_shape: NULL output");
  if (!dtype_ok(in_dtype)) return fail(RA_ERR_UNSUPPORTED, "ra_tile_shape: bad dtype %d", in_dtype);
  if (D != 64 && D != 128) return fail(RA_ERR_UNSUPPORTED, "ra_tile_shape: D=%lld", (long long)D);
  *block_m = in_dtype == RA_BF16 ? ra::kBf16BlockM : ra::kF32BlockM;
  *block_n = in_dtype == RA_BF16 ? ra::kBf16BlockN : ra::kF32BlockN;
  return ok();
}

int ra_block_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                      int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D, int in_dtype,
                      int o_dtype, int causal, const ra_shard* q_sh, const ra_shard* kv_sh,
                      float scale, hipStream_t stream) {
  int rc = check_dims(B, H, Sq, Sk, D);
  if (rc) return rc;
  if ((rc = check_kv_heads(H, H_kv))) return rc;
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype))
    return fail(RA_ERR_UNSUPPORTED, "dtype (%d, %d) not RA_F32/RA_BF16", in_dtype, o_dtype);
  if (causal) {
    if ((rc = check_shard(q_sh, Sq, "q_sh"))) return rc;
    if ((rc = check_shard(kv_sh, Sk, "kv_sh"))) return rc;
  }
  if (isnan(scale) || isinf(scale)) return fail(RA_ERR_INVALID_ARG, "scale is not finite");
  const bool empty = B == 0 || H == 0 || Sq == 0;
  if (!empty) {
    if (!q || !o || !lse || (Sk > 0 && (!k || !v))) return fail(RA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (misaligned(q) || misaligned(o) || misaligned(lse) || (Sk > 0 && (misaligned(k) || misaligned(v))))
      return fail(RA_ERR_MISALIGNED, "tensor pointer not 16-byte aligned");
  }
  if (empty) return ok();

  ra::AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.k[0] = k;
  a.v[0] = v;
  a.o = o;
  a.lse = lse;
  a.B = (int32_t)B;
  a.H = (int32_t)H;
  a.Hkv = (int32_t)H_kv;
  a.Sq = (int32_t)Sq;
  a.Sk = (int32_t)Sk;
  a.nsteps = Sk > 0 ? 1 : 0;
  a.causal = causal ? 1 : 0;
  a.store_final = 1;
  a.scale = scale > 0.f ? scale : (float)(1.0 / sqrt((double)D));
  if (causal) {
    a.qpos = to_pos(*q_sh);
    a.kv_assign = kv_sh->assign;
    a.kv_world = kv_sh->world;
    a.kv_len = kv_sh->global_len;
    a.kv_rank[0] = kv_sh->rank;
  }
  return launch_attn(a, (int)D, in_dtype, o_dtype, stream);
}

size_t ra_ring_share_workspace_bytes(int64_t B, int64_t H, int64_t S_loc, int64_t D) {
  if (B < 0 || H < 0 || S_loc < 0 || D < 0) return 0;
  return (size_t)4 * (size_t)(B * S_loc * H * D) + (size_t)16 * (size_t)(B * H * S_loc);
}

}  // extern "C"

namespace {

// ra_ring_share, with the debug tile counter of the instrumented kernel when dbg is not null.
int ring_share_impl(const void* q, const void* const* k_shares, const void* const* v_shares, void* o,
                    float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t S_loc, int64_t D, int N,
                    int rank, int assign, int causal, int in_dtype, int o_dtype, float scale,
                    int start_step, int num_steps, void* ws, size_t ws_bytes, int32_t* dbg,
                    hipStream_t stream) {
  int rc = check_dims(B, H, S_loc, S_loc, D);
  if (rc) return rc;
  if ((rc = check_kv_heads(H, H_kv))) return rc;
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype))
    return fail(RA_ERR_UNSUPPORTED, "dtype (%d, %d) not RA_F32/RA_BF16", in_dtype, o_dtype);
  if (N < 1) return fail(RA_ERR_INVALID_ARG, "ring size N=%d < 1", N);
  if (N > RA_MAX_WORLD) return fail(RA_ERR_UNSUPPORTED, "ring size N=%d > %d", N, RA_MAX_WORLD);
  if (rank < 0 || rank >= N) return fail(RA_ERR_INVALID_ARG, "rank %d not in [0, %d)", rank, N);
  if (assign < RA_CONTIGUOUS || assign > RA_ZIGZAG) return fail(RA_ERR_INVALID_ARG, "unknown assignment %d", assign);
  if (start_step < 0 || num_steps < 1 || start_step + num_steps > N)
    return fail(RA_ERR_INVALID_ARG, "step range [%d, %d) not inside [0, %d] or empty", start_step,
                start_step + num_steps, N);
  if (isnan(scale) || isinf(scale)) return fail(RA_ERR_INVALID_ARG, "scale is not finite");
  const int64_t L = (int64_t)N * S_loc;
  if (L >= ((int64_t)1 << 31)) return fail(RA_ERR_UNSUPPORTED, "global length N*S_loc = %lld >= 2^31", (long long)L);
  if (causal && assign == RA_ZIGZAG && S_loc % 2)
    return fail(RA_ERR_SHAPE, "zigzag needs L %% 2N == 0 (S_loc=%lld is odd)", (long long)S_loc);
  const bool load_state = start_step > 0;
  const bool store_final = start_step + num_steps == N;
  const bool empty = B == 0 || H == 0 || S_loc == 0;
  if (!empty) {
    if (!q || !k_shares || !v_shares) return fail(RA_ERR_INVALID_ARG, "NULL q or share array");
    for (int i = 0; i < N; ++i) {
      if (!k_shares[i] || !v_shares[i]) return fail(RA_ERR_INVALID_ARG, "share %d pointer is NULL", i);
      if (misaligned(k_shares[i]) || misaligned(v_shares[i]))
        return fail(RA_ERR_MISALIGNED, "share %d pointer not 16-byte aligned", i);
    }
    if (misaligned(q)) return fail(RA_ERR_MISALIGNED, "q not 16-byte aligned");
    if (store_final) {
      if (!o || !lse) return fail(RA_ERR_INVALID_ARG, "NULL o or lse");
      if (misaligned(o) || misaligned(lse)) return fail(RA_ERR_MISALIGNED, "o/lse not 16-byte aligned");
    }
    if (load_state || !store_final) {
      if (!ws) return fail(RA_ERR_INVALID_ARG, "workspace needed to %s the running state",
                           load_state ? "resume" : "keep");
      if (misaligned(ws)) return fail(RA_ERR_MISALIGNED, "workspace not 16-byte aligned");
      if (ws_bytes < ra_ring_share_workspace_bytes(B, H, S_loc, D))
        return fail(RA_ERR_INVALID_ARG, "workspace %zu bytes < %zu needed", ws_bytes,
                    ra_ring_share_workspace_bytes(B, H, S_loc, D));
    }
  }
  if (empty) return ok();

  const float scale_eff = scale > 0.f ? scale : (float)(1.0 / sqrt((double)D));
  WsTag tag;
  memset(&tag, 0, sizeof tag);
  tag.in_dtype = in_dtype;
  tag.assign = assign;
  tag.causal = causal ? 1 : 0;
  tag.N = N;
  tag.rank = rank;
  tag.B = B;
  tag.H = H;
  tag.H_kv = H_kv;
  tag.S = S_loc;
  tag.D = D;
  memcpy(&tag.scale_bits, &scale_eff, sizeof scale_eff);
  if (load_state) {
    tag.next_step = start_step;
    if ((rc = check_resume(ws, tag))) return rc;
  }

  ra::AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = q;
  for (int st = 0; st < num_steps; ++st) {
    // Ring order ([Digest] §3.1/§3.3): at step s the rank holds the KV of rank (rank - s) mod N.
    const int s = start_step + st;
    const int src = ((rank - s) % N + N) % N;
    a.k[st] = k_shares[src];
    a.v[st] = v_shares[src];
    a.kv_rank[st] = src;
  }
  a.o = o;
  a.lse = lse;
  if (ws) {
    // [B, S, H, D] fp32 O, then [B, H, S] fp64 running max, then [B, H, S] fp64 running sum.
    // The O part is a multiple of 16 bytes (D is 64 or 128), so the fp64 parts stay aligned.
    float* w = (float*)ws;
    a.ws_o = w;
    a.ws_m = (double*)(w + B * S_loc * H * D);
    a.ws_l = a.ws_m + B * H * S_loc;
  }
  a.B = (int32_t)B;
  a.H = (int32_t)H;
  a.Hkv = (int32_t)H_kv;
  a.Sq = (int32_t)S_loc;
  a.Sk = (int32_t)S_loc;
  a.nsteps = num_steps;
  a.causal = causal ? 1 : 0;
  a.load_state = load_state ? 1 : 0;
  a.store_final = store_final ? 1 : 0;
  a.scale = scale_eff;
  a.qpos = ra::make_pos(assign, N, rank, L);
  a.kv_assign = assign;
  a.kv_world = N;
  a.kv_len = L;
  a.dbg_counts = dbg;
  if ((rc = launch_attn(a, (int)D, in_dtype, o_dtype, stream))) return rc;
  if (!store_final) {
    tag.next_step = start_step + num_steps;
    record_state(ws, tag);
  }
  return ok();
}

}  // namespace

extern "C" {

int ra_ring_share(const void* q, const void* const* k_shares, const void* const* v_shares, void* o,
                  float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t S_loc, int64_t D, int N,
                  int rank, int assign, int causal, int in_dtype, int o_dtype, float scale,
                  int start_step, int num_steps, void* ws, size_t ws_bytes, hipStream_t stream) {
  return ring_share_impl(q, k_shares, v_shares, o, lse, B, H, H_kv, S_loc, D, N, rank, assign, causal,
                         in_dtype, o_dtype, scale, start_step, num_steps, ws, ws_bytes, nullptr, stream);
}

int64_t ra_debug_tile_count_slots(int64_t B, int64_t H, int64_t S_loc) {
  if (B < 0 || H < 0 || S_loc < 0) return 0;
  return (S_loc + ra::kBf16BlockM - 1) / ra::kBf16BlockM * B * H * 32;
}

int ra_debug_tile_counts(const void* q, const void* const* k_shares, const void* const* v_shares, void* o,
                         float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t S_loc, int64_t D, int N,
                         int rank, int assign, int causal, int o_dtype, float scale, int32_t* counts,
                         int64_t counts_len, hipStream_t stream) {
  if (B < 0 || H < 0 || S_loc < 0) return fail(RA_ERR_INVALID_ARG, "negative size");
  const int64_t need = ra_debug_tile_count_slots(B, H, S_loc);
  if (need > 0) {
    if (!counts) return fail(RA_ERR_INVALID_ARG, "NULL counts buffer");
    if (misaligned(counts)) return fail(RA_ERR_MISALIGNED, "counts not 16-byte aligned");
    if (counts_len < need)
      return fail(RA_ERR_INVALID_ARG, "counts holds %lld slots, %lld needed", (long long)counts_len, (long long)need);
  }
  return ring_share_impl(q, k_shares, v_shares, o, lse, B, H, H_kv, S_loc, D, N, rank, assign, causal, RA_BF16,
                         o_dtype, scale, 0, N, nullptr, 0, counts, stream);
}

size_t ra_ring_share_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S_loc) {
  if (B < 0 || H < 0 || S_loc < 0) return 0;
  return (size_t)8 * (size_t)(B * H * S_loc);
}

}  // extern "C"

namespace {

// ra_ring_share_bwd with the Delta buffer either from the caller's workspace (noalloc == false)
// or the library's static device scratch (noalloc == true; ws is ignored).
int ring_share_bwd_impl(const void* q, const void* const* k_shares, const void* const* v_shares,
                        const void* o, const float* lse, const void* dout, float* dq,
                        float* const* dk_shares, float* const* dv_shares, int64_t B, int64_t H,
                        int64_t H_kv, int64_t S_loc, int64_t D, int N, int rank, int assign, int causal,
                        int in_dtype, float scale, void* ws, size_t ws_bytes, bool noalloc, hipStream_t stream) {
  int rc = check_dims(B, H, S_loc, S_loc, D);
  if (rc) return rc;
  if ((rc = check_kv_heads(H, H_kv))) return rc;
  if (in_dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "backward runs on bf16 inputs only (in_dtype %d)", in_dtype);
  if (N < 1) return fail(RA_ERR_INVALID_ARG, "ring size N=%d < 1", N);
  if (N > RA_MAX_WORLD) return fail(RA_ERR_UNSUPPORTED, "ring size N=%d > %d", N, RA_MAX_WORLD);
  if (rank < 0 || rank >= N) return fail(RA_ERR_INVALID_ARG, "rank %d not in [0, %d)", rank, N);
  if (assign < RA_CONTIGUOUS || assign > RA_ZIGZAG) return fail(RA_ERR_INVALID_ARG, "unknown assignment %d", assign);
  if (isnan(scale) || isinf(scale)) return fail(RA_ERR_INVALID_ARG, "scale is not finite");
  const int64_t L = (int64_t)N * S_loc;
  if (L >= ((int64_t)1 << 31)) return fail(RA_ERR_UNSUPPORTED, "global length N*S_loc = %lld >= 2^31", (long long)L);
  if (causal && assign == RA_ZIGZAG && S_loc % 2)
    return fail(RA_ERR_SHAPE, "zigzag needs L %% 2N == 0 (S_loc=%lld is odd)", (long long)S_loc);
  const bool empty = B == 0 || H == 0 || S_loc == 0;
  if (empty) return ok();
  if (!q || !o || !lse || !dout || !dq || !k_shares || !v_shares || !dk_shares || !dv_shares)
    return fail(RA_ERR_INVALID_ARG, "NULL tensor pointer or share array");
  if (misaligned(q) || misaligned(o) || misaligned(lse) || misaligned(dout) || misaligned(dq))
    return fail(RA_ERR_MISALIGNED, "tensor pointer not 16-byte aligned");
  for (int i = 0; i < N; ++i) {
    if (!k_shares[i] || !v_shares[i] || !dk_shares[i] || !dv_shares[i])
      return fail(RA_ERR_INVALID_ARG, "share %d pointer is NULL", i);
    if (misaligned(k_shares[i]) || misaligned(v_shares[i]) || misaligned(dk_shares[i]) || misaligned(dv_shares[i]))
      return fail(RA_ERR_MISALIGNED, "share %d pointer not 16-byte aligned", i);
  }
  if (noalloc) {
    if (ra_ring_share_bwd_workspace_bytes(B, H, S_loc) > (size_t)RA_BWD_NOALLOC_MAX_BYTES)
      return fail(RA_ERR_UNSUPPORTED, "B*H*S_loc = %lld rows' terms need %zu bytes, above the %d-byte device scratch",
                  (long long)(B * H * S_loc), ra_ring_share_bwd_workspace_bytes(B, H, S_loc),
                  RA_BWD_NOALLOC_MAX_BYTES);
    float* p = nullptr;
    hipError_t e = ra::bwd_scratch(&p);
    if (e != hipSuccess) return fail(RA_ERR_HIP, "device scratch lookup failed: %s", hipGetErrorString(e));
    ws = p;
  } else {
    if (!ws) return fail(RA_ERR_INVALID_ARG, "workspace needed for the row terms");
    if (misaligned(ws)) return fail(RA_ERR_MISALIGNED, "workspace not 16-byte aligned");
    if (ws_bytes < ra_ring_share_bwd_workspace_bytes(B, H, S_loc))
      return fail(RA_ERR_INVALID_ARG, "workspace %zu bytes < %zu needed", ws_bytes,
                  ra_ring_share_bwd_workspace_bytes(B, H, S_loc));
  }

  ra::BwdArgs a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.delta = (float*)ws;
  a.lse2 = a.delta + B * H * S_loc;
  a.dq = dq;
  for (int s = 0; s < N; ++s) {
    const int src = ((rank - s) % N + N) % N;  // ring order, as in the forward
    a.k[s] = k_shares[src];
    a.v[s] = v_shares[src];
    a.dk[s] = dk_shares[src];
    a.dv[s] = dv_shares[src];
    a.kv_rank[s] = src;
  }
  a.B = (int32_t)B;
  a.H = (int32_t)H;
  a.Hkv = (int32_t)H_kv;
  a.Sq = (int32_t)S_loc;
  a.Sk = (int32_t)S_loc;
  a.nsteps = N;
  a.causal = causal ? 1 : 0;
  a.scale = scale > 0.f ? scale : (float)(1.0 / sqrt((double)D));
  a.qpos = ra::make_pos(assign, N, rank, L);
  a.kv_assign = assign;
  a.kv_world = N;
  a.kv_len = L;
  hipError_t e = ra::launch_attn_bwd(a, (int)D, stream);
  if (e != hipSuccess) return fail(RA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int ra_ring_share_bwd(const void* q, const void* const* k_shares, const void* const* v_shares,
                      const void* o, const float* lse, const void* dout, float* dq,
                      float* const* dk_shares, float* const* dv_shares, int64_t B, int64_t H,
                      int64_t H_kv, int64_t S_loc, int64_t D, int N, int rank, int assign, int causal,
                      int in_dtype, float scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  return ring_share_bwd_impl(q, k_shares, v_shares, o, lse, dout, dq, dk_shares, dv_shares, B, H, H_kv, S_loc, D, N,
                             rank, assign, causal, in_dtype, scale, ws, ws_bytes, false, stream);
}

int ra_ring_share_bwd_noalloc(const void* q, const void* const* k_shares, const void* const* v_shares,
                              const void* o, const float* lse, const void* dout, float* dq,
                              float* const* dk_shares, float* const* dv_shares, int64_t B, int64_t H,
                              int64_t H_kv, int64_t S_loc, int64_t D, int N, int rank, int assign,
                              int causal, int in_dtype, float scale, hipStream_t stream) {
  return ring_share_bwd_impl(q, k_shares, v_shares, o, lse, dout, dq, dk_shares, dv_shares, B, H, H_kv, S_loc, D, N,
                             rank, assign, causal, in_dtype, scale, nullptr, 0, true, stream);
}

int ra_lse_merge(void* o_acc, float* lse_acc, const void* o_blk, const float* lse_blk, int64_t B,
                 int64_t H, int64_t S, int64_t D, int acc_dtype, int blk_dtype, hipStream_t stream) {
  if (B < 0 || H < 0 || S < 0 || D < 0) return fail(RA_ERR_INVALID_ARG, "negative size");
  if (!dtype_ok(acc_dtype) || !dtype_ok(blk_dtype))
    return fail(RA_ERR_UNSUPPORTED, "dtype (%d, %d) not RA_F32/RA_BF16", acc_dtype, blk_dtype);
  if (D == 0 || D % 8) return fail(RA_ERR_UNSUPPORTED, "D=%lld must be a positive multiple of 8", (long long)D);
  if (B * S * H == 0) return ok();
  if (!o_acc || !lse_acc || !o_blk || !lse_blk) return fail(RA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (misaligned(o_acc) || misaligned(o_blk) || ((uintptr_t)lse_acc & 3) || ((uintptr_t)lse_blk & 3))
    return fail(RA_ERR_MISALIGNED, "tensor pointer misaligned");
  hipError_t e = ra::launch_lse_merge(o_acc, lse_acc, o_blk, lse_blk, B, H, S, D, acc_dtype, blk_dtype, stream);
  if (e != hipSuccess) return fail(RA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

int ra_seq2head_permute_n(const void* const* ins, void* const* outs, int n_tensors, int64_t B, int64_t P,
                          int64_t S_loc, int64_t H, int64_t D, int dtype, int dst_rank, int inverse,
                          hipStream_t stream) {
  if (B < 0 || S_loc < 0 || H < 0 || D < 0) return fail(RA_ERR_INVALID_ARG, "negative size");
  if (P < 1) return fail(RA_ERR_INVALID_ARG, "P=%lld < 1", (long long)P);
  if (n_tensors < 0 || n_tensors > RA_MAX_PERMUTE)
    return fail(RA_ERR_INVALID_ARG, "n_tensors=%d not in [0, %d]", n_tensors, RA_MAX_PERMUTE);
  if (!dtype_ok(dtype)) return fail(RA_ERR_UNSUPPORTED, "dtype %d not RA_F32/RA_BF16", dtype);
  if (H % P) return fail(RA_ERR_SHAPE, "P=%lld does not divide H=%lld", (long long)P, (long long)H);
  if (dst_rank < -1 || dst_rank >= P)
    return fail(RA_ERR_INVALID_ARG, "dst_rank %d not in [-1, %lld)", dst_rank, (long long)P);
  if (B * S_loc * H * D == 0 || n_tensors == 0) return ok();
  if (!ins || !outs) return fail(RA_ERR_INVALID_ARG, "NULL tensor array");
  for (int i = 0; i < n_tensors; ++i) {
    if (!ins[i] || !outs[i]) return fail(RA_ERR_INVALID_ARG, "tensor %d pointer is NULL", i);
    if (misaligned(ins[i]) || misaligned(outs[i]))
      return fail(RA_ERR_MISALIGNED, "tensor %d pointer not 16-byte aligned", i);
  }
  hipError_t e = ra::launch_permute(ins, outs, n_tensors, B, P, S_loc, H, D, dtype == RA_BF16 ? 2 : 4, dst_rank,
                                    inverse ? 1 : 0, stream);
  if (e != hipSuccess) return fail(RA_ERR_HIP, "permute launch failed: %s", hipGetErrorString(e));
  return ok();
}

int ra_seq2head_permute(const void* in, void* out, int64_t B, int64_t P, int64_t S_loc, int64_t H,
                        int64_t D, int dtype, int dst_rank, int inverse, hipStream_t stream) {
  const void* ins[1] = {in};
  void* outs[1] = {out};
  return ra_seq2head_permute_n(ins, outs, 1, B, P, S_loc, H, D, dtype, dst_rank, inverse, stream);
}

int ra_share_work(const ra_shard* q_sh, const ra_shard* kv_sh, int64_t Sq, int64_t Sk, int causal,
                  int64_t block_m, int64_t block_n, int64_t out[4]) {
  if (!out) return fail(RA_ERR_INVALID_ARG, "NULL output");
  if (Sq < 0 || Sk < 0 || block_m < 1 || block_n < 1) return fail(RA_ERR_INVALID_ARG, "bad sizes");
  int rc;
  if (causal) {
    if ((rc = check_shard(q_sh, Sq, "q_sh"))) return rc;
    if ((rc = check_shard(kv_sh, Sk, "kv_sh"))) return rc;
  }
  const int64_t n_qt = (Sq + block_m - 1) / block_m;
  const int64_t n_kt = (Sk + block_n - 1) / block_n;
  if (!causal) {
    out[0] = Sq * Sk;
    out[1] = n_qt * n_kt;
    out[2] = out[3] = 0;
    return ok();
  }
  const ra::Pos qp = to_pos(*q_sh), kp = to_pos(*kv_sh);
  int64_t pairs = 0;
  for (int64_t i = 0; i < Sq; ++i) pairs += ra::clamp64(ra::count_le(kp, ra::pos_of(qp, (int32_t)i)), 0, Sk);
  int64_t full = 0, partial = 0, skip = 0;
  for (int64_t t = 0; t < n_qt; ++t) {
    const int64_t r0 = t * block_m, r1 = (r0 + block_m < Sq ? r0 + block_m : Sq) - 1;
    const int64_t cmin = ra::clamp64(ra::count_le(kp, ra::pos_of(qp, (int32_t)r0)), 0, Sk);
    const int64_t cmax = ra::clamp64(ra::count_le(kp, ra::pos_of(qp, (int32_t)r1)), 0, Sk);
    // Tiles made only of keys visible to the tile's first (smallest-position) row are full.
    const int64_t nfull = cmin / block_n + ((cmin == Sk && Sk % block_n) ? 1 : 0);
    const int64_t active = (cmax + block_n - 1) / block_n;
    full += nfull;
    partial += active - nfull;
    skip += n_kt - active;
  }
  out[0] = pairs;
  out[1] = full;
  out[2] = partial;
  out[3] = skip;
  return ok();
}

int ra_debug_positions(const ra_shard* sh, int64_t* out, hipStream_t stream) {
  int rc = check_shard(sh, -1, "sh");
  if (rc) return rc;
  const int64_t n = sh->global_len / sh->world;
  if (n == 0) return ok();
  if (!out) return fail(RA_ERR_INVALID_ARG, "NULL output");
  hipError_t e = ra::launch_debug_positions(to_pos(*sh), n, out, stream);
  if (e != hipSuccess) return fail(RA_ERR_HIP, "positions launch failed: %s", hipGetErrorString(e));
  return ok();
}

int ra_debug_mask(const ra_shard* q_sh, const ra_shard* kv_sh, int64_t Sq, int64_t Sk, uint8_t* out,
                  hipStream_t stream) {
  int rc;
  if ((rc = check_shard(q_sh, Sq, "q_sh"))) return rc;
  if ((rc = check_shard(kv_sh, Sk, "kv_sh"))) return rc;
  if (Sq * Sk == 0) return ok();
  if (!out) return fail(RA_ERR_INVALID_ARG, "NULL output");
  hipError_t e = ra::launch_debug_mask(to_pos(*q_sh), to_pos(*kv_sh), Sq, Sk, out, stream);
  if (e != hipSuccess) return fail(RA_ERR_HIP, "mask launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
