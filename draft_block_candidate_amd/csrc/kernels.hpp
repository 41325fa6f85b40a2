// Kernel launchers (host-callable), one translation unit per kernel family.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ll {

hipError_t launch_weights_init(void* dst, uint64_t numel, uint64_t key, int kind, float scale,
                               hipStream_t stream);

// a1: fused log-partition + exact top-K. part_* are scratch of the sizes in
// topk_ws_layout(); outputs topk_idx/topk_logp [rows, K], lse [rows] (may be null).
// merge = false with rows split into P > 1 chunks leaves the chunk outputs
// in part_* for launch_node_build_merge (topk_idx / topk_logp / lse unwritten).
hipError_t launch_topk_lse(const void* logits, int rows, int V, int K, int dtype, float* part_val,
                           int32_t* part_idx, float* part_ms, int32_t* topk_idx, float* topk_logp,
                           float* lse, hipStream_t stream, bool merge = true);

// a1 over one shard of a split vocabulary: the shard's [rows, V] slice holds
// ids id_offset .. id_offset + V - 1. Outputs per row the shard's K best
// (value, global id) pairs and its (max, sum of exp(x - max)) pair:
// out_val/out_idx [rows, K], out_ms [rows, 2]; part_* are chunk scratch of
// topk_ws_layout(rows, V, K).
hipError_t launch_topk_shard(const void* logits, int rows, int V, int K, int dtype, int id_offset,
                             float* part_val, int32_t* part_idx, float* part_ms, float* out_val,
                             int32_t* out_idx, float* out_ms, hipStream_t stream);
// Merge of G shard outputs stacked [G, rows, K] / [G, rows, 2] (shards in
// ascending order of their id ranges) into topk_idx, topk_logp, lse.
hipError_t launch_topk_merge_shards(int G, int rows, int K, const float* val, const int32_t* idx,
                                    const float* ms, int32_t* topk_idx, float* topk_logp,
                                    float* lse, hipStream_t stream);

// a2: node features, confidence MLP layer 1 and the embedding/slot/rank sum.
//   hid  bf16 [M, H] = bf16(silu(W1c f + b1c));  xbase float [M, H] = (E[tok] + S[s]) + R[j]
// With ph set (the paper's head): only slots 1..B-1 (M = N (B-1) K) and
// xbase = (ph[n B + s] + S[s]) + R[j], ph the projected drafter states [N B, H].
// xbase may be null (lattice head only): then only hid is written and the
// table sum is left to the next linear's epilogue (NodeSource).
// Lattice head with rows split into 1 < P <= 64 chunks and either fewer than
// 4,096 tokens or K = 8 (H <= 2048): the node build of the lattice head (hidden activations only) that
// also merges each token's row from the top-K chunk outputs (part_* as
// launch_topk_lse(..., merge = false) leaves them) and writes topk_idx,
// topk_logp and, if given, lse, as the merge kernel would.
bool node_build_merges(int N, int B, int K, int H, int P);
hipError_t launch_node_build_merge(const float* part_val, const int32_t* part_idx, const float* part_ms,
                                   int P, int32_t* topk_idx, float* topk_logp, float* lse, int N, int B,
                                   int K, int H, const uint16_t* conf_w1, const float* conf_b1,
                                   uint16_t* hid, int V, hipStream_t stream);
hipError_t launch_node_build(const int32_t* topk_idx, const float* topk_logp, int N, int B, int K,
                             int H, const uint16_t* E, const float* ph, const uint16_t* S,
                             const uint16_t* R, const uint16_t* conf_w1, const float* conf_b1,
                             uint16_t* hid, float* xbase, int V, hipStream_t stream);

// The paper's head (paper_head.hip).
//   gather_rows: out [N (B-1) K, Ht] = table[token] of the drafted candidates
//   rmsnorm_bf16: out = bf16(RMSNorm(x)) for bf16 rows x [M, H] (H % 8 == 0, H <= 8192)
//   concat: out [N P, 3H] = [u, tb[n], bf16(u * tb[n])], P lattice rows per block
//   anchor_rows: slot 0 of outv/inv [N, B, K, d_e]: out rows = unit(apre[n]),
//                in rows = 0 (d_e <= 1024)
hipError_t launch_gather_rows(const int32_t* topk_idx, int N, int B, int K, const uint16_t* table,
                              int Ht, int V, uint16_t* out, hipStream_t stream);
hipError_t launch_rmsnorm_bf16(const uint16_t* x, int M, int H, const float* gamma, float eps,
                               uint16_t* out, hipStream_t stream);
hipError_t launch_concat(const uint16_t* u, const uint16_t* tb, int N, int per_block, int H,
                         uint16_t* out, hipStream_t stream);
hipError_t launch_anchor_rows(const float* apre, int N, int B, int K, int de, uint16_t* outv,
                              uint16_t* inv, hipStream_t stream);

enum Epilogue { EPI_F32 = 0, EPI_BF16 = 1, EPI_SILU_BF16 = 2, EPI_RESID_F32 = 3 };

// Schedule of one linear layer: split = 1 for one pass over K, else the number
// of K slices; part_floats is the fp32 scratch it needs (zero if none).
struct GemmPlan {
  int bm, bn, ks, split, tiles;
  size_t part_floats;
};
GemmPlan plan_linear(int M, int Kd, int N);
// True when launch_linear runs the product as one few-row pass over K
// (no split-K scratch) for epilogues that need no whole rows.
bool uses_skinny(int M, int Kd, int N);

// Residual of the node build: the residual of row m is not read from memory
// but formed from the tables, ((E[tok[m]] + S[s]) + R[j]) in float32 with
// m = (n B + s) K + j (the lattice head's table sum, added in the order the
// node is written); the confidence network's output is then added to it.
struct NodeSource {
  const int32_t* tok = nullptr;   // [M] token ids (the top-K ids)
  const uint16_t *E = nullptr, *S = nullptr, *R = nullptr;   // bf16 tables, rows of N
  int K = 1, B = 1, V = 1;        // candidates per slot, slots per block, rows of E
  uint64_t magic_k = 0, magic_b = 0;   // div_magic(K), div_magic(B)
};
// floor(m / d) for any 32-bit m and 1 <= d <= 64 as (m * ceil(2^38 / d)) >> 38
// (the round-up multiplier with 6 extra bits is exact for 32-bit numerators),
// evaluated in 64-bit pieces.
__host__ __device__ inline uint64_t div_magic(int d) { return ((1ull << 38) + (uint64_t)d - 1) / (uint64_t)d; }
__host__ __device__ inline uint32_t div_by(uint32_t m, uint64_t magic) {
  const uint64_t lo = magic & 0xffffffffull, hi = magic >> 32;
  return (uint32_t)(((uint64_t)m * hi + (((uint64_t)m * lo) >> 32)) >> 6);
}

// What follows the product y = A W^T + bias:
//   kind       EPI_* store of y (EPI_RESID_F32: out = resid + y)
//   norm_out   if set (with EPI_RESID_F32): also u = bf16(RMSNorm(out; norm_gamma, eps))
//   heads_out  if set (with EPI_F32, N = 2 d_e): unit-normalised bf16 halves to
//              heads_out / heads_in (out then receives y only when not split);
//              with heads_group > 0, row m lands in row
//              m + (m / heads_group + 1) heads_skip of heads_out / heads_in
struct LinearEpilogue {
  int kind = EPI_F32;
  const float* resid = nullptr;
  const float* norm_gamma = nullptr;
  float eps = 0.f;
  uint16_t* norm_out = nullptr;
  uint16_t* heads_out = nullptr;
  uint16_t* heads_in = nullptr;
  int heads_group = 0, heads_skip = 0;
  // EPI_RESID_F32 only: the residual comes from the node tables instead of
  // `resid` (see NodeSource); allowed where linear_takes_node_source() holds
  const NodeSource* node = nullptr;
};
// True when launch_linear forms a residual-plus-RMSNorm epilogue (EPI_RESID_F32
// with norm_out) of an M x Kd -> N product in a kernel that can take the node
// tables as its residual (the many-row DMA kernel, the split-K row reduce).
bool linear_takes_node_source(int M, int Kd, int N);

// Destination row of the out/in heads' row m (see LinearEpilogue).
__host__ __device__ inline int64_t heads_row(int64_t m, int group, int skip) {
  return group > 0 ? m + (m / group + 1) * skip : m;
}

// Y = A[M,Kd] W[N,Kd]^T + bias with the epilogue above (bf16 in, fp32
// accumulate, MFMA). part: fp32 scratch of plan_linear(M, Kd, N).part_floats.
hipError_t launch_linear(const uint16_t* A, int M, int Kd, const uint16_t* W, int N,
                         const float* bias, const LinearEpilogue& ep, void* out, float* part,
                         hipStream_t stream);

hipError_t launch_rmsnorm(const float* x, int M, int H, const float* gamma, float eps,
                          uint16_t* out, hipStream_t stream);

// Few-row lattices (65..128 tokens, d_h = 128, fewer than 2,048 rows, a head
// count the split-K reduce is built for): attention and the output
// projection's per-head split-K slices in one launch. part: [heads][M][H]
// fp32, M = N B K; the attention output is not written. Reduce with
// launch_splitk_reduce(heads, ...).
bool attention_o_fusable(int N, int B, int K, int H, int heads);
hipError_t launch_attention_o(const uint16_t* qkv, int N, int B, int K, int H, int heads,
                              const float* dist, const float* same, const uint16_t* wo, float* part,
                              hipStream_t stream);
// The split-K reduce of launch_linear for S given slices part[S][M][N] with
// the epilogue ep (S in {2, 3, 4, 6, 8, 12, 16}).
hipError_t launch_splitk_reduce(int S, int M, int N, const float* bias, const LinearEpilogue& ep,
                                void* out, const float* part, hipStream_t stream);
hipError_t launch_attention(const uint16_t* qkv, int N, int B, int K, int H, int heads,
                            const float* dist, const float* same, uint16_t* out,
                            hipStream_t stream);


hipError_t launch_pair_scores(const uint16_t* outv, const uint16_t* inv, int N, int B, int K,
                              int d_e, float* cos, hipStream_t stream);

// Commit rule of a6: greedy walk, exact best path, or sampled commit.
enum CommitKind { RULE_GREEDY = 0, RULE_EXACT = 1, RULE_SAMPLE = 2 };
struct CommitRule {
  int kind = RULE_GREEDY;
  float alpha = 1.f;
  int use_logp = 1;
  const float* temperature = nullptr;  // [N] (RULE_SAMPLE; T <= 0: greedy row)
  const float* uniforms = nullptr;     // [N, B] in [0, 1) (RULE_SAMPLE)
  float* proposal = nullptr;           // [N, B, K] (RULE_SAMPLE; may be null)
};

// Fused a5 + a6 (cosines in LDS; cos_out may be null). With cos_in set, the
// cosines [N, B-1, K, K] are read instead of computed (outv/inv unused); with
// cos_slices > 1 they are the sum, in slice order, of cos_slices such arrays
// stored one after another (the partial products of launch_pair_slices).
// Needs scores_walk_lds_bytes(B, K) <= kScoresWalkMaxLds.
constexpr size_t kScoresWalkMaxLds = 128 * 1024;
size_t scores_walk_lds_bytes(int B, int K);
hipError_t launch_scores_walk(const uint16_t* outv, const uint16_t* inv, const float* cos_in,
                              int cos_slices, const int32_t* topk_idx, const float* topk_logp,
                              int N, int B, int K, int d_e, const CommitRule& rule, float* cos_out,
                              int32_t* out_tokens, float* score, float* gap, hipStream_t stream);

// Pair cosines of wide vectors in 256-wide slices of d_e: part holds
// pair_slice_count(d_e) arrays [N, B-1, K, K] of partial sums.
// From d_e = 256 the rerank path forms the cosines this way (one wave per
// pair and slice instead of one workgroup per block).
constexpr int kPairSliceMinDe = 256;
inline int pair_slice_count(int d_e) { return (d_e + 255) / 256; }
hipError_t launch_pair_slices(const uint16_t* outv, const uint16_t* inv, int N, int B, int K,
                              int d_e, float* part, hipStream_t stream);

hipError_t launch_greedy_walk(const int32_t* topk_idx, const float* topk_logp, const float* cos,
                              int N, int B, int K, float alpha, int use_logp, int32_t* out_tokens,
                              float* score, float* gap, hipStream_t stream);

// Diagnostic: shader-clock probe. out[0] = ticks of the 100 MHz constant
// counter over a window of window_ticks of them, out[1] = shader-clock cycles
// (s_memtime) over the same window; out is device uint64 [2].
hipError_t launch_clock_probe(uint64_t* out, uint64_t window_ticks, hipStream_t stream);

}  // namespace ll
