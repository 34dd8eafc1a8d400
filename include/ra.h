/*
 * ra.h -- C ABI of the per-device Ring Attention inner loop for MI355X (gfx950).
 *
 * Pages this interface follows (cited by title and section):
 *   [Digest] "从 Ring Attention 到 DeepSpeed Ulysses，再到 USP 统一框架" (jsqmd.com digest)
 *   [Notes]  "主流序列并行(SP)方案对比 + 大模型通信原语" (hzhuang.org notes)
 *   [Q14]    "序列并行（Sequence Parallelism）解决了什么问题？和 TP 是什么关系？" (playoffer)
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library never
 *     allocates, frees or keeps caller memory. The one exception is the ring call's
 *     k_shares / v_shares: HOST arrays holding N device pointers.
 *   - Q, K, V, O are [B, S, H, D] row-major with D contiguous (the [bs, seq, heads,
 *     head_dim] layout of the pages' ring example, [Digest] §10). LSE is fp32
 *     [B, H, S], natural log.
 *   - Every call enqueues work on the caller's stream and returns at once; nothing
 *     synchronises the device. A fault inside a kernel surfaces at the caller's next
 *     synchronisation.
 *   - Arguments are validated on the host before anything is launched, so every
 *     error code below is produced without touching the GPU. Calls return RA_OK or a
 *     negative status; ra_last_error() then describes the failure (a thread-local
 *     string owned by the library, valid until the next call on the same thread).
 *   - Nothing throws across the ABI. Calls on different streams may run concurrently
 *     as long as they do not write the same memory.
 *   - Device pointers must be 16-byte aligned (128-bit loads and stores).
 *   - Empty inputs (B, H or a sequence length of 0) are valid and launch nothing.
 *   - Environment: RA_KV_SPLIT selects the workgroup layout of the bf16 attention
 *     kernel. Unset or "auto": when one workgroup per 128-row query tile would leave a
 *     compute unit with fewer than two workgroups, each query tile's key tiles are
 *     split between two groups of waves of one workgroup and their states merged at the
 *     end; "always" / "never" force either layout. Results agree to rounding (the
 *     order in which key tiles are folded differs); read at every launch.
 *   - Environment: RA_PAIR_TILES. Unset or "auto": for causal calls on striped K/V
 *     shares whose grid still gives two workgroups per compute unit when halved, one
 *     workgroup takes the query tiles n-1-p and p (the second walked backward over its
 *     key tiles); "always" pairs every causal call with two or more query tiles (unless
 *     the key split applies), "never" keeps one tile per workgroup. Results agree to
 *     rounding either way; read at every launch.
 *   - Environment: RA_PAIR_GROUP. Paired workgroups visit a step's key tiles in groups (tiles
 *     of one step, then the same range of the next step): of 8 tiles for K/V shares of at most
 *     8192 rows, of 32 otherwise; "short" / "long" force 8 / 32. Results agree to rounding.
 */
#ifndef RA_H_
#define RA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define RA_OK 0
#define RA_ERR_INVALID_ARG (-1)  /* null pointer, rank >= N, N < 1, negative size, bad step range */
#define RA_ERR_UNSUPPORTED (-2)  /* dtype not in {RA_F32, RA_BF16}, D not in {64, 128}, N > RA_MAX_WORLD,
                                    sizes beyond the 32-bit indexing limits (see the calls) */
#define RA_ERR_SHAPE (-3)        /* H % P != 0, L % N != 0, L % 2N != 0 (zigzag), sizes disagree */
#define RA_ERR_MISALIGNED (-4)   /* a device pointer is not 16-byte aligned */
#define RA_ERR_HIP (-5)          /* a HIP launch error */

#define RA_MAX_WORLD 64          /* largest ring size N accepted by ra_ring_share */
#define RA_MAX_PERMUTE 8         /* most tensors one ra_seq2head_permute_n call moves */
#define RA_BWD_NOALLOC_MAX_BYTES (16 << 20)  /* device scratch of ra_ring_share_bwd_noalloc */

typedef enum { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* Token -> rank assignment of a sequence of global_len tokens over world ranks.
 *   RA_CONTIGUOUS: rank r holds tokens [r*L/N, (r+1)*L/N)        ([Digest] §3.4, §4 listing)
 *   RA_STRIPED:    token t lives on rank t mod N                  ([Digest] §4)
 *   RA_ZIGZAG:     2N equal chunks; rank r holds chunks r, 2N-1-r ([Digest] §6 item 1)
 * Local row i of a share is the i-th smallest global position the rank holds. */
typedef enum { RA_CONTIGUOUS = 0, RA_STRIPED = 1, RA_ZIGZAG = 2 } ra_assign;

typedef struct {
  int32_t assign;      /* ra_assign */
  int32_t world;       /* N >= 1 */
  int32_t rank;        /* 0 <= rank < N */
  int64_t global_len;  /* L; L % N == 0 (L % 2N == 0 for zigzag) */
} ra_shard;

/*
 * ra_block_attn_fwd -- one ring step's block attention: local Q against one KV block
 * ("flash_attn_block(Q_local, K, V) -> (out, lse)" in the ring loop of [Digest] §3.3;
 * the definition softmax(Q K^T / sqrt(d)) V is [Digest] §2).
 *
 *   q     [B, Sq, H, D]  in_dtype           k, v  [B, Sk, H_kv, D]  in_dtype
 *   o     [B, Sq, H, D]  o_dtype (output)   lse   [B, H, Sq]     fp32 (output)
 *   H_kv: KV heads, 1 <= H_kv, H_kv dividing H (grouped-query attention: [Digest] §5.3 has
 *     GQA models with fewer KV heads than query heads, MQA with one); query head h attends
 *     KV head h / (H / H_kv). H_kv = H is plain multi-head attention. H_kv < 1 returns
 *     RA_ERR_INVALID_ARG, a non-divisor RA_ERR_SHAPE (ignored when H == 0).
 *   causal: if non-zero, key j is visible to query i iff pos_kv(j) <= pos_q(i), the
 *     positions coming from q_sh / kv_sh (the mask is taken by global position,
 *     [Q14] engineering notes; diagonal included, [Digest] §3.4). Then Sq must equal
 *     q_sh->global_len / q_sh->world and Sk likewise for kv_sh. If zero, every key is
 *     visible and q_sh / kv_sh may be NULL.
 *   scale: logit scale; <= 0 selects 1/sqrt(D) (softmax_scale=None, [Digest] §10).
 * Output: O normalised, LSE = ln(sum over visible keys of exp(scale * q.k)). A row with
 * no visible key gets O = 0 and LSE = -inf.
 * in_dtype RA_BF16 runs bf16 MFMA with fp32 accumulation; RA_F32 runs fp32 FMA.
 * D must be 64 or 128. Sq and Sk may be any non-negative size (ragged tails are masked).
 * Global lengths (q_sh->global_len, kv_sh->global_len) must be below 2^31; B*H, Sq and Sk
 * below 2^30; H*D*2 below 2^24 (bytes of one K/V row, multiplied in 24 bits); ceil(Sq/64)*B*H
 * below 2^31 (the launch grid). Beyond these limits the call returns RA_ERR_UNSUPPORTED.
 */
int ra_block_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D,
                      int in_dtype, int o_dtype, int causal,
                      const ra_shard* q_sh, const ra_shard* kv_sh, float scale,
                      hipStream_t stream);

/*
 * ra_lse_merge -- merge a block result into an accumulated one, in place
 * ("online_softmax_merge" of [Digest] §3.3, "merge_lse" and its formula in [Digest] §6
 * item 3):
 *     lse = max(a, b) + log(1 + exp(-|a - b|));  O = O_acc e^(a - lse) + O_blk e^(b - lse)
 * with a = lse_acc, b = lse_blk, O's normalised. A side whose lse is -inf contributes
 * nothing; two empty sides give O = 0, lse = -inf.
 *   o_acc [B, S, H, D] acc_dtype (in/out)   lse_acc [B, H, S] fp32 (in/out)
 *   o_blk [B, S, H, D] blk_dtype            lse_blk [B, H, S] fp32
 * D may be any positive multiple of 8. Merges in any order give the same result up to
 * rounding ([Digest] §3.2).
 */
int ra_lse_merge(void* o_acc, float* lse_acc, const void* o_blk, const float* lse_blk,
                 int64_t B, int64_t H, int64_t S, int64_t D, int acc_dtype, int blk_dtype,
                 hipStream_t stream);

/* Bytes of workspace ra_ring_share needs to keep the running state between calls:
 * un-normalised fp32 O [B, S, H, D], then the running max and the running sum [B, H, S]
 * each in 8-byte (fp64) slots. */
size_t ra_ring_share_workspace_bytes(int64_t B, int64_t H, int64_t S_loc, int64_t D);

/*
 * ra_ring_share -- every ring step of one rank's share on one stream ([Digest] §3.1 and
 * the loop of §3.3): step s attends the local Q to the KV share of rank
 * src = (rank - s) mod N (round 0 is local; KV moves to rank+1), folding each block into
 * the running (m, l, O) by the online-softmax update of [Digest] §3.2.
 *   q                    [B, S_loc, H, D] in_dtype, rank's share
 *   k_shares, v_shares   HOST arrays of N device pointers; entry i is rank i's share
 *                        [B, S_loc, H_kv, D] in_dtype (H_kv as in ra_block_attn_fwd)
 *   o, lse               outputs as in ra_block_attn_fwd, written when the last step
 *                        (start_step + num_steps == N) has run
 *   assign, causal       token assignment of the global sequence (L = N * S_loc) and
 *                        whether the causal mask by global position applies
 *   start_step, num_steps  run steps [start_step, start_step + num_steps), in ring order
 *                        (with bf16 inputs one call folds the KV tiles of its steps in groups
 *                        of 32 tiles, 2048 keys, taken round-robin over the steps; the result
 *                        is the same up to rounding, and num_steps == 1 is one ring step)
 *   ws, ws_bytes         running state (size from ra_ring_share_workspace_bytes). May be
 *                        NULL when start_step == 0 and num_steps == N (the state then stays
 *                        in registers). A call that ends before step N stores the state in
 *                        ws; a call with start_step > 0 resumes from it. The state is
 *                        opaque (its layout depends on in_dtype) and valid only for the same
 *                        q, in_dtype, scale, shape, assignment, mask, N and rank. The library
 *                        records these (on the host, per workspace address) for every call
 *                        that stores a state, and a resume returns RA_ERR_INVALID_ARG when
 *                        ws holds no state stored in this process, when any of them differs,
 *                        or when start_step is not the step the stored state ends at.
 * The result does not depend on how the N steps are split across calls, up to rounding.
 */
int ra_ring_share(const void* q, const void* const* k_shares, const void* const* v_shares,
                  void* o, float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t S_loc,
                  int64_t D, int N, int rank, int assign, int causal, int in_dtype, int o_dtype,
                  float scale, int start_step, int num_steps, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/* Bytes of workspace ra_ring_share_bwd needs: the row terms Delta [B, H, S] and the LSE in log2
 * units [B, H, S], both fp32. */
size_t ra_ring_share_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S_loc);

/*
 * ra_ring_share_bwd -- gradients of ra_ring_share's output. The pages train with ring
 * attention ([Digest] §3.1-§3.4) but print no backward formulas; this is the derivative of
 * the forward definition ([Digest] §2 with the causal matrix of §3.4) using the forward's
 * saved LSE: P = exp(scale q.k - LSE), Delta = rowsum(dO * O), dS = P (dO.v - Delta),
 * dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
 *   q, o, dout           [B, S_loc, H, D] bf16: the rank's Q share, the forward output and
 *                        the gradient of the loss with respect to it
 *   lse                  [B, H, S_loc] fp32: the forward LSE (natural log)
 *   k_shares, v_shares   HOST arrays of N device pointers, [B, S_loc, H_kv, D] bf16, as in
 *                        ra_ring_share
 *   dq                   [B, S_loc, H, D] fp32 output: gradient with respect to q
 *   dk_shares, dv_shares HOST arrays of N device pointers, [B, S_loc, H_kv, D] fp32 outputs:
 *                        entry i receives the gradient with respect to rank i's K and V
 *                        share from this rank's queries (on a real ring these travel back to
 *                        rank i and are summed over ranks); every entry is written
 *   H_kv, assign, causal, scale  as in ra_ring_share (scale <= 0 selects 1/sqrt(D))
 *   ws, ws_bytes         workspace, at least ra_ring_share_bwd_workspace_bytes(B, H, S_loc)
 * in_dtype must be RA_BF16 (RA_F32 returns RA_ERR_UNSUPPORTED); D is 64 or 128; size limits
 * and error codes as in ra_ring_share. Every ring step is taken in one call.
 */
int ra_ring_share_bwd(const void* q, const void* const* k_shares, const void* const* v_shares,
                      const void* o, const float* lse, const void* dout, float* dq,
                      float* const* dk_shares, float* const* dv_shares, int64_t B, int64_t H,
                      int64_t H_kv, int64_t S_loc, int64_t D, int N, int rank, int assign,
                      int causal, int in_dtype, float scale, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * ra_ring_share_bwd_noalloc -- ra_ring_share_bwd for callers that cannot allocate device memory
 * (code being captured into a HIP graph, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without ws / ws_bytes, the same kernels and the same results. The row terms
 * (what ra_ring_share_bwd keeps in its workspace) live in a static device array of
 * RA_BWD_NOALLOC_MAX_BYTES (16 MiB) that the library holds on every device it runs on until the
 * process ends; the call allocates and frees nothing. Limit:
 * ra_ring_share_bwd_workspace_bytes(B, H, S_loc) = 8 * B * H * S_loc <= RA_BWD_NOALLOC_MAX_BYTES,
 * i.e. B * H * S_loc <= 2,097,152, else RA_ERR_UNSUPPORTED (before anything is launched). Every call on a device uses that device's one array, so calls that overlap on one
 * device (concurrent streams, or threads without ordering) race and may return wrong gradients;
 * order them. The array needs no clearing: each call writes every row term before reading it.
 */
int ra_ring_share_bwd_noalloc(const void* q, const void* const* k_shares, const void* const* v_shares,
                              const void* o, const float* lse, const void* dout, float* dq,
                              float* const* dk_shares, float* const* dv_shares, int64_t B, int64_t H,
                              int64_t H_kv, int64_t S_loc, int64_t D, int N, int rank, int assign,
                              int causal, int in_dtype, float scale, hipStream_t stream);

/*
 * ra_seq2head_permute -- the local data movement of the Ulysses all-to-all ([Digest] §5.1,
 * [Notes] §3): sequence-sharded [bs, L/P, H, d] on each of P ranks to head-sharded
 * [bs, L, H/P, d], rank p taking heads [p*H/P, (p+1)*H/P), its full sequence ordered by
 * source rank.
 *   forward (inverse == 0): in  = [P, B, S_loc, H, D] (the P ranks' shares, stacked)
 *       dst_rank >= 0: out = [B, P*S_loc, H/P, D],
 *                      out[b, src*S_loc + s, h', :] = in[src, b, s, dst_rank*H/P + h', :]
 *       dst_rank == -1: out = [P, B, P*S_loc, H/P, D], every rank's result stacked
 *   inverse (inverse != 0): in = the forward output for dst_rank (or the stack for -1),
 *       out = [P, B, S_loc, H, D]; writes only the head slice(s) of dst_rank (all for -1)
 *       and leaves the other heads of out untouched.
 * dtype gives the element size (RA_BF16: 2 bytes, RA_F32: 4); the copy is bit-exact.
 * H % P != 0 is RA_ERR_SHAPE (the head-count constraint of [Digest] §5.3).
 */
int ra_seq2head_permute(const void* in, void* out, int64_t B, int64_t P, int64_t S_loc,
                        int64_t H, int64_t D, int dtype, int dst_rank, int inverse,
                        hipStream_t stream);

/*
 * ra_seq2head_permute_n -- ra_seq2head_permute of n_tensors tensors of the same shape and dtype
 * in one launch (the Q, K and V of a Ulysses step: [Digest] §5.1 sends all three through the
 * all-to-all). ins / outs are HOST arrays of n_tensors device pointers; tensor i is permuted from
 * ins[i] into outs[i] exactly as ra_seq2head_permute(ins[i], outs[i], ...) would. 0 <= n_tensors
 * <= RA_MAX_PERMUTE (else RA_ERR_INVALID_ARG); other arguments and errors as ra_seq2head_permute.
 */
int ra_seq2head_permute_n(const void* const* ins, void* const* outs, int n_tensors, int64_t B,
                          int64_t P, int64_t S_loc, int64_t H, int64_t D, int dtype, int dst_rank,
                          int inverse, hipStream_t stream);

/* Thread-local description of the last failure on this thread ("" after success). */
const char* ra_last_error(void);

/*
 * Planner and debug hooks.
 *
 * ra_share_work (host only, no GPU): causal work of one Q share against one KV share,
 * from the same position functions the kernels use. out[0] = visible (query, key) pairs,
 * out[1..3] = full / partial / skip tiles of block_m x block_n over [Sq, Sk] (a tile is
 * full when every existing pair in it is visible, skip when none is). Attention FLOPs are
 * 4 * D * out[0] per (batch, head). Returns a status like the calls above.
 */
int ra_share_work(const ra_shard* q_sh, const ra_shard* kv_sh, int64_t Sq, int64_t Sk,
                  int causal, int64_t block_m, int64_t block_n, int64_t out[4]);

/* Tile shape (rows of Q, keys of K/V) the attention kernel uses for in_dtype and D. */
int ra_tile_shape(int in_dtype, int64_t D, int64_t* block_m, int64_t* block_n);

/* Device: out[i] = global position of local row i of sh's share (i < L/N), int64. */
int ra_debug_positions(const ra_shard* sh, int64_t* out, hipStream_t stream);

/* Device: out[i*Sk + j] = 1 if key j of kv_sh's share is visible to query i of q_sh's
 * share under the causal mask, else 0; evaluated by the kernels' own mask function. */
int ra_debug_mask(const ra_shard* q_sh, const ra_shard* kv_sh, int64_t Sq, int64_t Sk,
                  uint8_t* out, hipStream_t stream);

/*
 * Device-side tile counts (debug hook, not part of the hot path). Tile skipping is what makes
 * causal work about half of the full product (the lower-triangular causal matrix of [Digest]
 * §3.4): these calls show which K/V tiles the bf16 kernel actually visits.
 *
 * ra_debug_tile_count_slots: int32 slots ra_debug_tile_counts writes for a share of S_loc query
 * rows: ceil(S_loc / block_m) * B * H * 32 (block_m from ra_tile_shape, 128 for bf16).
 *
 * ra_debug_tile_counts: the same computation and outputs as ra_ring_share over every ring step
 * (start_step 0, num_steps N, no workspace) with bf16 inputs, run through a copy of the bf16
 * kernel that also counts, for every wave, the K/V tiles (block_n = 64 keys) it folds into its
 * 32 query rows and, among those, the tiles on which it evaluates the mask (a tile is masked by
 * a wave when it is the ragged last tile of a share or when the wave's first query row does not
 * see the tile's last key). The workgroup layout (one query tile, key split, paired tiles) is
 * chosen exactly as for ra_ring_share. Output counts, int32 [ceil(S_loc/128), B, H, 8, 4]:
 * [qt, b, h, w, 0] = tiles folded in by wave slot w of query tile qt, [.., 1] = tiles it masked,
 * [.., 2] = bounds faults: tiles the wave copied or folded whose (step, tile) cursor lies outside
 * the call's steps or past the step's last visible tile or the share's end, [.., 3] = skip
 * faults: tiles it folded whose first key no query row of the query tile sees (causal). The
 * two fault counts are zero for a correct kernel; they are checked, not asserted, so a fault
 * is reported through the counts and never stops the kernel.
 * Wave slots 0-3 are the four waves of the first (or only) wave group, 4-7 those of the second
 * group of a key-split workgroup (zero otherwise); a wave whose rows all lie past S_loc counts
 * nothing. counts is a device buffer of counts_len >= ra_debug_tile_count_slots(..) slots,
 * 16-byte aligned; every slot is written. Other arguments and errors as in ra_ring_share.
 */
int64_t ra_debug_tile_count_slots(int64_t B, int64_t H, int64_t S_loc);
int ra_debug_tile_counts(const void* q, const void* const* k_shares, const void* const* v_shares,
                         void* o, float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t S_loc,
                         int64_t D, int N, int rank, int assign, int causal, int o_dtype, float scale,
                         int32_t* counts, int64_t counts_len, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RA_H_ */
