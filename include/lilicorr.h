/*
 * lilicorr.h - C ABI of the MI355X (gfx950) LiLiCorr reranking library.
 *
 * The library implements the inference path of the LiLiCorr candidate-lattice
 * reranker ("LiLiCorr: Lightweight Likelihood Correlation of Parallel Drafts
 * for Speculative Decoding", arXiv 2608.20530; serving kernels described in
 * the SGLang pull request "[Spec] Add LiLiCorr: a candidate-lattice reranker
 * for DFlash drafts"):
 *
 *   per-slot log-softmax + top-K  ->  one candidate-encoder pass emitting unit
 *   in/out vectors  ->  batched K x K cosine scores per adjacent slot pair  ->
 *   greedy left-to-right commit.
 *
 * Conventions shared by every entry point
 *   - Pointers named dev_* or documented as "device" are HIP device pointers;
 *     all others are host pointers.
 *   - Every buffer is owned by the caller. The library allocates no memory and
 *     keeps no mutable global state apart from a once-per-device architecture
 *     check.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     null stream) and the call returns after enqueueing. Outputs are valid
 *     once the stream has reached that point. No call synchronises the device.
 *   - Every function returning int returns LILICORR_OK (0) or a negative
 *     lilicorr_status. Argument checks run on the host before any launch; on
 *     an error nothing is enqueued and no output is touched.
 *   - Calls that share a workspace must not overlap; distinct workspaces make
 *     calls independent. Every entry point can be captured in a HIP graph (no
 *     memset nodes, no host synchronisation, fixed launch sequence).
 *   - Logits must be finite; this is not checked on the device.
 */
#ifndef LILICORR_H_
#define LILICORR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define LILICORR_API __attribute__((visibility("default")))
#else
#define LILICORR_API
#endif

#define LILICORR_ABI_VERSION 3u
#define LILICORR_MAX_SLOTS 64     /* B: slots per block */
#define LILICORR_MAX_TOPK 64      /* K: candidates per slot (one per wave lane) */
#define LILICORR_MAX_LATTICE 512  /* T = B*K tokens per block */

typedef enum {
  LILICORR_OK = 0,
  LILICORR_EINVAL = -1,       /* bad size, null required pointer, bad abi_version */
  LILICORR_EUNSUPPORTED = -2, /* dtype or geometry outside what the kernels build for, or device is not gfx950 */
  LILICORR_EWORKSPACE = -3,   /* workspace missing or smaller than lilicorr_workspace_bytes() */
  LILICORR_EWEIGHTS = -4,     /* weight descriptor does not match dims/vocabulary, or blob too small */
  LILICORR_EHIP = -5,         /* a HIP runtime call or kernel launch failed */
  LILICORR_ETOOLARGE = -6     /* lilicorr_rerank_noalloc: workspace need above its fixed scratch */
} lilicorr_status;

typedef enum { LILICORR_F32 = 0, LILICORR_BF16 = 1 } lilicorr_dtype;

/* Commit rule of the last step (all three score a step alike:
 * z_s(i, j) = fl32(logp[s][j] + fl32(alpha * cos_s[i][j])), or fl32(alpha * cos_s[i][j])
 * when use_logp = 0; slot 0 commits its top candidate, c_0 = 0).
 *   GREEDY  LiLiCorr paper, Section 3.5, Eq. (8): c_s = lowest j maximising z_s(c_{s-1}, j).
 *   EXACT   Appendix E, Eq. (12): the path maximising g(c) = sum_s z_s(c_{s-1}, c_s), summed
 *           left to right in fp32 and found by dynamic programming; every maximum (best
 *           predecessor, best final candidate) takes the lowest index, so among equal totals
 *           the path smallest when read from the last slot backward is returned.
 *   SAMPLE  SGLang PR, "Sampling the committed path (opt-in)": block n draws slot s from
 *           softmax(z_s(c_{s-1}, .) / T_n) by inverse CDF with the caller's uniform u[n, s]:
 *           c_s = number of cumulative sums C_j <= u * S (S the fp32 sum of the exps in
 *           ascending j), at most K - 1. Blocks with T_n <= 0 are greedy rows: the GREEDY
 *           path bit for bit, with one-hot proposals. */
typedef enum { LILICORR_RULE_GREEDY = 0, LILICORR_RULE_EXACT = 1, LILICORR_RULE_SAMPLE = 2 } lilicorr_rule;

/* Encoder geometry. LiLiCorr paper, Appendix A "Architecture" and Table 4:
 * a two-layer bidirectional transformer of width `hidden` with `heads`
 * attention heads and feed-forward width `ffn`; in/out vectors of width d_e.
 * Supported: layers == 2; hidden % 64 == 0; ffn % 64 == 0; d_e % 32 == 0;
 * hidden / heads in {32, 64, 128}; hidden <= 4096; ffn <= 16384; d_e <= 1024.
 *
 * target_hidden = 0 selects the lattice head over all B slots whose node embeds
 * the token with its own table E (no drafter or target inputs). target_hidden
 * > 0 selects the paper's own head (Section 3.2, Appendix A): the lattice holds
 * the B-1 drafted slots; a node sums the target's frozen input embedding of the
 * token projected down (E_t, width target_hidden), the drafter's hidden state
 * at its slot projected down (width drafter_hidden), the confidence network and
 * the slot/rank tables; after the transformer each node is fused with the
 * projected target state (concat [node, t', node * t'] -> linear -> SiLU); a
 * third head gives the anchor's (slot 0's) out vector from t'. Then 64 <=
 * target_hidden <= 8192, 64 <= drafter_hidden <= 16384, both multiples of 64. */
typedef struct {
  int32_t hidden, heads, ffn, d_e, layers;
  int32_t target_hidden;   /* H_t; 0 = lattice head */
  int32_t drafter_hidden;  /* H_d (paper head only) */
} lilicorr_dims;

/* Encoder weights: a device blob of lilicorr_weights_bytes() bytes filled by
 * lilicorr_weights_init() from (dims, vocab, seed). The pages publish no
 * trained head, so the weights are seeded random with a counter-based
 * SplitMix64 stream (layout and values: lilicorr_weights_tensor()). */
typedef struct {
  lilicorr_dims dims;
  int32_t vocab;   /* V: rows of the token embedding table */
  uint64_t seed;
  void* dev;       /* device pointer, 256-byte aligned, caller-owned */
  size_t bytes;    /* size of the blob at dev */
} lilicorr_weights;

/* Stages of lilicorr_rerank, for the optional timing events below. The five
 * per-layer stages of layer l are LILICORR_STAGE_QKV + 5*l .. FFN2 + 5*l. */
typedef enum {
  LILICORR_STAGE_TOPK = 0,         /* fused log-partition + top-K (and its chunk merge) */
  LILICORR_STAGE_NODE = 1,         /* embedding gathers + first confidence-MLP layer */
  LILICORR_STAGE_CONF_LINEAR = 2,  /* second confidence-MLP layer, residual, RMSNorm */
  LILICORR_STAGE_QKV = 3,          /* layer 0: fused q|k|v projection */
  LILICORR_STAGE_ATTENTION = 4,    /* layer 0: lattice attention */
  LILICORR_STAGE_O = 5,            /* layer 0: output projection, residual, RMSNorm */
  LILICORR_STAGE_FFN1 = 6,         /* layer 0: first FFN linear + SiLU */
  LILICORR_STAGE_FFN2 = 7,         /* layer 0: second FFN linear, residual, RMSNorm */
  LILICORR_STAGE_HEADS = 13,       /* out|in heads + unit normalisation */
  LILICORR_STAGE_SCORES_WALK = 14, /* pair scores + greedy walk */
  LILICORR_STAGE_COUNT = 15
} lilicorr_stage;

typedef struct {
  uint32_t abi_version;            /* must be LILICORR_ABI_VERSION */
  int32_t num_blocks;              /* N independent draft blocks (>= 1) */
  int32_t logits_dtype;            /* lilicorr_dtype of the logits */
  float alpha;                     /* weight of the cosine term in the commit rule */
  int32_t use_logp;                /* 1: z = logp + alpha*cos; 0: z = alpha*cos (paper's sigma*cos) */
  const lilicorr_weights* weights; /* host pointer to an initialised descriptor */
  void* workspace;                 /* device scratch, >= lilicorr_workspace_bytes() */
  size_t workspace_bytes;
  void* stream;                    /* hipStream_t */
  /* Optional device outputs, NULL = not written:
   *   dbg_topk_idx  int32  [N,B,K]   vocabulary ids, (logit desc, id asc)
   *   dbg_topk_logp float  [N,B,K]   fl32(x - fl32(lse))
   *   dbg_lse       float  [N,B]     log sum_v exp(x_v)
   *   dbg_outv/inv  bf16   [N,B,K,d_e] unit out / in vectors (raw uint16 bits)
   *   dbg_cos       float  [N,B-1,K,K] cos_s[a][b] = out[s-1,a] . in[s,b]
   *   dbg_score     float  [N,B]     committed score per slot (slot 0: its top logp)
   *   dbg_gap       float  [N,B]     committed score minus best other score (0 at slot 0 / K=1) */
  int32_t* dbg_topk_idx;
  float* dbg_topk_logp;
  float* dbg_lse;
  uint16_t* dbg_outv;
  uint16_t* dbg_inv;
  float* dbg_cos;
  float* dbg_score;
  float* dbg_gap;
  /* Optional timing of one stage (measurement only). When timing_begin and
   * timing_end are both non-NULL (hipEvent_t handles created by the caller),
   * they are recorded on `stream` right before the first and right after the
   * last kernel of stage `timing_stage` (a lilicorr_stage value, < COUNT).
   * Both NULL: nothing is recorded and timing_stage is ignored. */
  int32_t timing_stage;
  void* timing_begin;
  void* timing_end;
  /* Commit rule (lilicorr_rule). For LILICORR_RULE_SAMPLE:
   *   temperature  device float [N]     per-block temperature (<= 0: greedy row), required
   *   uniforms     device float [N, B]  draws in [0, 1), slot 0 unused, required
   *   proposal     device float [N, B, K] distribution each slot was drawn from (may be NULL)
   * Other rules ignore the three pointers. dbg_score then holds z along the committed path;
   * dbg_gap is the runner-up gap for greedy steps and 0 for exact or drawn steps. */
  int32_t rule;
  const float* temperature;
  const float* uniforms;
  float* proposal;
  /* Inputs of the paper's head (dims.target_hidden > 0; ignored otherwise), required:
   *   hidden  device bf16 bits [N, B, drafter_hidden]  drafter hidden state per slot (slot 0 unused)
   *   target  device bf16 bits [N, target_hidden]      target state behind the block's anchor
   * With this head slot 0 is the anchor: its out vectors (dbg_outv) all hold the anchor
   * head's vector, its in vectors are zero, and the walk starts from its candidate 0. The
   * paper's commit rule is use_logp = 0 with alpha = sigma = 8 (Table 4). */
  const uint16_t* hidden;
  const uint16_t* target;
} lilicorr_params;

/* The whole reranking path (LiLiCorr paper, Section 3.5 "Single-pass
 * decoding"; commit by p->rule, see lilicorr_rule).
 *   logits      device, [N, B, V] row-major (V contiguous), dtype p->logits_dtype
 *   B, V, K     slots per block (1..64), vocabulary (K..2^31-1), candidates (1..64), B*K <= 512
 *   out_tokens  device int32 [N, B]: committed vocabulary id per slot
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EWEIGHTS (host checks), EHIP. */
LILICORR_API int lilicorr_rerank(const void* logits, int B, int V, int K, const lilicorr_params* p,
                    int32_t* out_tokens);

/* Allocation-free variant of lilicorr_rerank, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, outputs and launch sequence
 * as lilicorr_rerank, except that p->workspace / p->workspace_bytes are ignored:
 * the workspace is a fixed array of LILICORR_NOALLOC_SCRATCH_BYTES in the
 * library's device code, one per device, held until the process ends. The call
 * allocates nothing (its first call on a device only looks the array's address
 * up, so make that first call outside graph capture). Nothing in it needs to
 * start at zero (lilicorr_rerank_audit: every region is written before it is
 * read). Every call on a device shares that device's array: calls that overlap
 * on one device (concurrent streams, or other host threads) race and must be
 * serialised by the caller; a call's results are its outputs, not the array.
 * Errors: those of lilicorr_rerank except EWORKSPACE, plus ETOOLARGE when
 * lilicorr_workspace_bytes(N, B, V, K, dims) exceeds the array (host check, nothing
 * launched): 1-4 blocks of the 1024-wide encoder at K = 8, one block at K = 16,
 * one block of the paper's head at its Table 4 size. */
#define LILICORR_NOALLOC_SCRATCH_BYTES (48u << 20)
LILICORR_API int lilicorr_rerank_noalloc(const void* logits, int B, int V, int K,
                                         const lilicorr_params* p, int32_t* out_tokens);

/* Host-only audit of lilicorr_rerank's launch sequence for N blocks of B slots,
 * vocabulary V, K candidates and the given geometry (the commit rule and the
 * debug outputs do not change which workspace regions are used). Launches
 * nothing and needs no GPU. Each launch declares the workspace regions it reads
 * and writes (the split-K and top-K chunk scratch are written and read inside
 * their own launch); the audit walks the sequence in launch order and fails at
 * the first launch that reads a region no earlier launch has written, so a
 * workspace of any prior contents (lilicorr_rerank never clears it) gives the
 * same result. drop_step >= 0 leaves that launch out of the walk (a test of the
 * audit itself: a dropped producer must be caught).
 *   report  host buffer (may be NULL) for one line per launch:
 *           "<index> <name> reads <regions> writes <regions>", and
 *           " UNWRITTEN <regions>" on the failing line; NUL-terminated, truncated
 *           to report_bytes.
 * Returns OK, EINVAL (bad sizes, or a read before any write), EUNSUPPORTED (dims). */
LILICORR_API int lilicorr_rerank_audit(int N, int B, int V, int K, const lilicorr_dims* dims,
                                       int drop_step, char* report, size_t report_bytes);

/* Host-only check of lilicorr_rerank's arguments; launches nothing and needs no GPU.
 * Returns exactly the status lilicorr_rerank would return before launching. */
LILICORR_API int lilicorr_validate(const void* logits, int B, int V, int K, const lilicorr_params* p,
                      const int32_t* out_tokens);

/* Workspace bytes lilicorr_rerank needs for N blocks of B slots, vocabulary V,
 * K candidates and the given geometry. Host only; 0 if the sizes are invalid. */
LILICORR_API size_t lilicorr_workspace_bytes(int N, int B, int V, int K, const lilicorr_dims* dims);

/* Bytes of the weight blob for (dims, V). Host only; 0 if invalid. */
LILICORR_API size_t lilicorr_weights_bytes(const lilicorr_dims* dims, int V);

/* Fill w->dev with the synthetic weights of (w->dims, w->vocab, w->seed).
 * Tensor t, row-major element e:  k_t = splitmix64(seed ^ (t << 40)),
 * r = splitmix64(k_t + e), u = (r >> 40) * 2^-24,
 * w = fl32((2u - 1) * fl32(1/sqrt(fan_in)))  (matrices rounded to bf16, RNE),
 * gains = fl32(1 + 0.25 (2u - 1)). splitmix64(x) is the first output of a
 * SplitMix64 generator with state x (Steele, Lea, Flood, OOPSLA 2014).
 * Errors: EINVAL, EUNSUPPORTED, EWEIGHTS (w->bytes too small), EHIP. */
LILICORR_API int lilicorr_weights_init(lilicorr_weights* w, void* stream);

/* Where tensor `id` lives in the weight blob: byte offset, element count and
 * storage dtype (LILICORR_BF16 or LILICORR_F32). Ids: 0 E[V,H], 1 S[64,H],
 * 2 R[64,H], 3 conf_w1[H,5], 4 conf_b1[H], 5 conf_w2[H,H], 6 conf_b2[H];
 * layer l (base 16+16l): +0 gamma1[H], +1 wqkv[3H,H], +2 bqkv[3H], +3 wo[H,H],
 * +4 bo[H], +5 gamma2[H], +6 w1[F,H], +7 b1[F], +8 w2[H,F], +9 b2[H],
 * +10 dist[heads,127], +11 same[heads]; 48 gamma_f[H], 49 w_out[d_e,H],
 * 50 b_out[d_e], 51 w_in[d_e,H], 52 b_in[d_e]. The paper's head (target_hidden
 * = H_t > 0, drafter_hidden = H_d) has no tensor 0 and adds 56 E_t[V,H_t],
 * 57 w_emb[H,H_t], 58 b_emb[H], 59 w_hid[H,H_d], 60 b_hid[H], 61 gamma_t[H_t],
 * 62 w_tgt[H,H_t], 63 b_tgt[H], 64 w_fuse[H,3H], 65 b_fuse[H], 66 w_anchor[d_e,H],
 * 67 b_anchor[d_e]. Host only. EINVAL if unknown. */
LILICORR_API int lilicorr_weights_tensor(const lilicorr_dims* dims, int V, int id, size_t* offset_bytes,
                            size_t* numel, int* dtype);

/* Status code to a static string. */
LILICORR_API const char* lilicorr_strerror(int code);

/* ---- Component entry points: single steps of the path, same kernels ---- */

/* Fused log-partition + exact top-K per row (SGLang PR, "Why the custom
 * kernels": one pass over [n, V] returning the top-k and the log-partition).
 *   logits     device [rows, V], dtype LILICORR_F32 or LILICORR_BF16
 *   topk_idx   device int32 [rows, K]  ids ordered by (logit desc, id asc)
 *   topk_logp  device float [rows, K]  fl32(x - fl32(lse))
 *   lse        device float [rows]     (may be NULL)
 *   workspace  device, >= lilicorr_topk_workspace_bytes(rows, V, K) */
LILICORR_API size_t lilicorr_topk_workspace_bytes(int rows, int V, int K);
LILICORR_API int lilicorr_topk_lse(const void* logits, int rows, int V, int K, int dtype, void* workspace,
                      size_t workspace_bytes, int32_t* topk_idx, float* topk_logp, float* lse,
                      void* stream);

/* Top-K of a vocabulary split across shards (a tensor-parallel LM head; the SGLang PR's
 * top-K + log-partition of "Why the custom kernels" for tp > 1): each shard reduces its
 * slice, then one merge over the shards' outputs gives lilicorr_topk_lse's result for
 * the whole rows (ids exactly; lse and logp to float32 rounding).
 *
 * Shard side. logits device [rows, V_shard] holds vocabulary ids id_offset ..
 * id_offset + V_shard - 1 of each row (K <= V_shard). Outputs (device, caller-owned):
 *   part_val  float [rows, K]  the slice's K best values, (value desc, id asc)
 *   part_idx  int32 [rows, K]  their global ids (id_offset added)
 *   part_ms   float [rows, 2]  (m, s): a reference m and s = sum_v exp(x_v - m) in fp32,
 *                              so the slice's log-partition is m + log s
 *   workspace device, >= lilicorr_topk_shard_workspace_bytes(rows, V_shard, K)
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP. */
LILICORR_API size_t lilicorr_topk_shard_workspace_bytes(int rows, int V_shard, int K);
LILICORR_API int lilicorr_topk_shard(const void* logits, int rows, int V_shard, int K, int dtype,
                                     int id_offset, void* workspace, size_t workspace_bytes,
                                     float* part_val, int32_t* part_idx, float* part_ms,
                                     void* stream);

/* Merge side. The G shard outputs stacked as part_val/part_idx [G, rows, K] and
 * part_ms [G, rows, 2] (device), the shards in ascending order of their id ranges (all
 * ids of shard g below those of shard g + 1), G in 1..64 -> topk_idx int32 [rows, K],
 * topk_logp float [rows, K], lse float [rows] (may be NULL), as lilicorr_topk_lse.
 * Errors: EINVAL, EHIP. */
LILICORR_API int lilicorr_topk_merge(const float* part_val, const int32_t* part_idx,
                                     const float* part_ms, int G, int rows, int K,
                                     int32_t* topk_idx, float* topk_logp, float* lse, void* stream);

/* Pair scores (LiLiCorr paper, Eq. (1) and Section 3.5: one product per
 * adjacent slot pair, batched over the block).
 *   outv, inv  device bf16 bits [N, B, K, d_e]; cos device float [N, B-1, K, K]. */
LILICORR_API int lilicorr_pair_scores(const uint16_t* outv, const uint16_t* inv, int N, int B, int K, int d_e,
                         float* cos, void* stream);

/* Greedy commit (LiLiCorr paper, Eq. (8); ties to the lower index as in the
 * SGLang PR). c_0 = 0; for s >= 1: z_j = fl32(logp[s][j] + fl32(alpha *
 * cos[s-1][c_{s-1}][j])) (use_logp = 1) or fl32(alpha * cos[..]) (use_logp = 0);
 * c_s = lowest j with maximal z_j; out_tokens[s] = topk_idx[s][c_s].
 *   topk_idx int32 / topk_logp float [N,B,K], cos float [N,B-1,K,K] (device)
 *   out_tokens int32 [N,B]; score, gap float [N,B] (device, may be NULL).
 * For B * K <= 512 this runs the commit kernel of lilicorr_rerank on the given
 * cosines; larger lattices (up to 64 x 64) run a one-wave-per-block walk over
 * the cosines in global memory. Errors: EINVAL, EHIP. */
LILICORR_API int lilicorr_greedy_walk(const int32_t* topk_idx, const float* topk_logp, const float* cos, int N,
                         int B, int K, float alpha, int use_logp, int32_t* out_tokens,
                         float* score, float* gap, void* stream);

/* Exact best path over given scores (LiLiCorr paper, Appendix E, Eq. (12); LILICORR_RULE_EXACT).
 *   topk_idx int32 / topk_logp float [N,B,K], cos float [N,B-1,K,K] (device)
 *   out_tokens int32 [N,B]; score float [N,B] (device, may be NULL): z along the path.
 * B * K <= 512. Errors: EINVAL, EUNSUPPORTED, EHIP. */
LILICORR_API int lilicorr_best_path(const int32_t* topk_idx, const float* topk_logp, const float* cos,
                                    int N, int B, int K, float alpha, int use_logp,
                                    int32_t* out_tokens, float* score, void* stream);

/* Sampled commit over given scores (SGLang PR, "Sampling the committed path (opt-in)" and
 * lilicorr_sample_path; LILICORR_RULE_SAMPLE). Arguments as lilicorr_best_path, plus
 *   temperature device float [N] (<= 0: greedy row), uniforms device float [N,B] in [0, 1),
 *   proposal device float [N,B,K] (may be NULL): softmax(z / T) each slot was drawn from.
 * B * K <= 512. Errors: EINVAL, EUNSUPPORTED, EHIP. */
LILICORR_API int lilicorr_sample_path(const int32_t* topk_idx, const float* topk_logp,
                                      const float* cos, int N, int B, int K, float alpha,
                                      int use_logp, const float* temperature,
                                      const float* uniforms, int32_t* out_tokens, float* proposal,
                                      float* score, void* stream);

/* One linear layer on MFMA: Y[M,N] = A[M,Kd] . W[N,Kd]^T + bias[N], bf16
 * inputs, fp32 accumulation, then the epilogue:
 *   0: out float  = y            1: out bf16 = bf16(y)
 *   2: out bf16   = bf16(silu(y)) 3: out float = resid + y (resid may equal out)
 * A, W: device bf16 bits; bias device float [N] (may be NULL = 0).
 * workspace: device scratch of lilicorr_linear_workspace_bytes(M, Kd, N) bytes
 * (split-K partial sums for few rows; may be NULL when that size is 256 or
 * less). Requires Kd % 64 == 0. */
LILICORR_API size_t lilicorr_linear_workspace_bytes(int M, int Kd, int N);
LILICORR_API int lilicorr_linear(const uint16_t* A, int M, int Kd, const uint16_t* W, int N,
                                 const float* bias, int epilogue, const float* resid, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* RMSNorm of fp32 rows then bf16 rounding: out = bf16(x / sqrt(mean(x^2) + eps) * gamma).
 * x device float [M, H]; gamma device float [H]; out device bf16 [M, H]. H % 64 == 0, H <= 8192. */
LILICORR_API int lilicorr_rmsnorm(const float* x, int M, int H, const float* gamma, float eps, uint16_t* out,
                     void* stream);

/* Lattice attention of one layer (LiLiCorr paper, Appendix A: bidirectional
 * over the whole lattice; per-head biases by signed slot distance and for
 * same-slot pairs). qkv device bf16 [N*T, 3H] (q | k | v, heads as contiguous
 * d_h column groups); T = B*K tokens per block, token t in slot t / K;
 * dist device float [heads, 127] indexed by slot_key - slot_query + 63;
 * same device float [heads]; out device bf16 [N*T, H] = bf16(softmax-weighted v)
 * with p = bf16(exp(s - rowmax)) and the row sum of the unrounded exp. */
LILICORR_API int lilicorr_lattice_attention(const uint16_t* qkv, int N, int B, int K, int hidden, int heads,
                               const float* dist, const float* same, uint16_t* out, void* stream);

/* Diagnostic, not part of the reranking path: the shader clock of the GPU
 * over a window. One wave reads the 100 MHz constant counter and the shader
 * clock counter at the start and the end of a window of window_us
 * microseconds (1 .. 1,000,000) of the constant counter, sleeping in between,
 * and writes out[0] = constant-counter ticks elapsed, out[1] = shader-clock
 * cycles elapsed (clock in GHz = 0.1 * out[1] / out[0]). Launched on its own
 * stream beside a running launch, it reads the clock that launch runs at.
 * out: device uint64 [2], 8-byte aligned, written by the probe. Errors: EINVAL
 * (null or misaligned out, window out of range), EUNSUPPORTED (not gfx950),
 * EHIP. */
LILICORR_API int lilicorr_clock_probe(uint64_t* out, int64_t window_us, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LILICORR_H_ */
