// C ABI of the library: argument checks, workspace carve-up and the launch
// sequence of the reranking path. See include/lilicorr.h for the contract.
#include <atomic>
#include <cstring>
#include <string>

#include "common.hpp"
#include "kernels.hpp"
#include "layout.hpp"
#include "lilicorr.h"

using namespace ll;

namespace {

constexpr float kRmsEps = 1e-6f;

bool dims_supported(const lilicorr_dims* d) {
  if (!d) return false;
  if (d->layers != 2) return false;
  if (d->hidden < 64 || d->hidden > 4096 || d->hidden % 64) return false;
  if (d->heads < 1 || d->hidden % d->heads) return false;
  const int dh = d->hidden / d->heads;
  if (dh != 32 && dh != 64 && dh != 128) return false;
  if (d->ffn < 64 || d->ffn > 16384 || d->ffn % 64) return false;
  if (d->d_e < 32 || d->d_e > 1024 || d->d_e % 32) return false;
  if (d->target_hidden != 0) {   // the paper's head
    if (d->target_hidden < 64 || d->target_hidden > 8192 || d->target_hidden % 64) return false;
    if (d->drafter_hidden < 64 || d->drafter_hidden > 16384 || d->drafter_hidden % 64) return false;
  } else if (d->drafter_hidden != 0) {
    return false;
  }
  return true;
}

bool sizes_ok(int N, int B, int V, int K) {
  if (N < 1 || B < 1 || B > LILICORR_MAX_SLOTS || K < 1 || K > LILICORR_MAX_TOPK) return false;
  if (V < K) return false;
  if (B * K > LILICORR_MAX_LATTICE) return false;
  // row-local indices and per-launch grid sizes stay within 32 bits
  if ((int64_t)N * B * K > (int64_t)1 << 30) return false;
  return true;
}

// gfx950 check, once per device (the code objects are built for gfx950 only).
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LILICORR_EHIP;
  if (dev < 0 || dev >= 64) return LILICORR_EUNSUPPORTED;
  int st = g_arch_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LILICORR_EHIP;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? LILICORR_OK : LILICORR_EUNSUPPORTED;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LILICORR_OK : LILICORR_EHIP; }

int validate_args(const void* logits, int B, int V, int K, const lilicorr_params* p,
                  const int32_t* out_tokens, bool with_workspace);

// Fixed device scratch of lilicorr_rerank_noalloc: the rerank workspace of
// callers that cannot allocate. Each device that runs the library holds its
// own copy for the life of the process. In host code `scratch` is only the
// symbol's host-side stand-in; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[LILICORR_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_dev[64];
std::atomic<int> g_scratch_lock{0};

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LILICORR_EHIP;
  if (dev < 0 || dev >= 64) return LILICORR_EUNSUPPORTED;
  void* ptr = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!ptr) {
    int expected = 0;
    while (!g_scratch_lock.compare_exchange_weak(expected, 1, std::memory_order_acquire)) expected = 0;
    ptr = g_scratch_dev[dev].load(std::memory_order_relaxed);
    hipError_t e = hipSuccess;
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e == hipSuccess && ptr) g_scratch_dev[dev].store(ptr, std::memory_order_release);
    }
    g_scratch_lock.store(0, std::memory_order_release);
    if (e != hipSuccess || !ptr) return LILICORR_EHIP;
  }
  *out = ptr;
  return LILICORR_OK;
}

CommitRule commit_rule(const lilicorr_params& p) {
  CommitRule r;
  r.kind = p.rule;
  r.alpha = p.alpha;
  r.use_logp = p.use_logp;
  r.temperature = p.temperature;
  r.uniforms = p.uniforms;
  r.proposal = p.proposal;
  return r;
}

// Shared checks of the stand-alone commit entry points that run the fused
// kernel on given cosines (its LDS holds one block's B-1 K x K matrices).
int commit_args_ok(const int32_t* topk_idx, const float* topk_logp, const float* cos, int N, int B,
                   int K, int use_logp, const int32_t* out_tokens) {
  if (!topk_idx || !topk_logp || !out_tokens || (B > 1 && !cos)) return LILICORR_EINVAL;
  if (N < 1 || B < 1 || B > LILICORR_MAX_SLOTS || K < 1 || K > LILICORR_MAX_TOPK ||
      B * K > LILICORR_MAX_LATTICE)
    return LILICORR_EINVAL;
  if (use_logp != 0 && use_logp != 1) return LILICORR_EINVAL;
  if (scores_walk_lds_bytes(B, K) > kScoresWalkMaxLds) return LILICORR_EUNSUPPORTED;
  return LILICORR_OK;
}

#define LL_TRY(expr)                                \
  do {                                              \
    hipError_t _e = (expr);                         \
    if (_e != hipSuccess) return LILICORR_EHIP;     \
  } while (0)

// Regions of the rerank workspace (rerank_ws_layout), as bits for the audit.
// outv / inv are split into slot 0's rows and the other slots' rows, which the
// paper's head writes in separate launches. o_part is the gemm_part memory
// while it carries the fused attention's per-head output-projection slices to
// the next launch (gemm_part itself is scratch within one linear's launches).
enum WsRegion {
  WS_TOPK_PART, WS_TOPK_IDX, WS_TOPK_LOGP, WS_X, WS_HID, WS_U, WS_QKV, WS_ATTN, WS_HEADS, WS_OUTV,
  WS_INV, WS_GEMM_PART, WS_PH, WS_AE, WS_TNORM, WS_TB, WS_APRE, WS_OUTV_SLOT0, WS_INV_SLOT0,
  WS_O_PART, WS_REGION_COUNT
};
#define WS_BIT(r) (1u << WS_##r)
const char* const kWsRegionName[WS_REGION_COUNT] = {
    "topk_part", "topk_idx", "topk_logp", "x", "hid", "u", "qkv", "attn", "heads", "outv",
    "inv", "gemm_part", "ph", "ae", "tnorm", "tb", "apre", "outv_slot0", "inv_slot0", "o_part"};

// Dry run of the launch sequence: each step states the workspace regions it
// reads and writes; a read of a region that no earlier step wrote fails.
// drop >= 0 leaves that step out (its writes never happen).
struct Audit {
  int drop = -1;
  int index = 0;
  uint32_t written = 0;
  std::string log;
  static std::string names(uint32_t m) {
    std::string r;
    for (int i = 0; i < WS_REGION_COUNT; ++i)
      if (m & (1u << i)) {
        if (!r.empty()) r += ",";
        r += kWsRegionName[i];
      }
    return r.empty() ? "-" : r;
  }
  int step(const char* name, uint32_t reads, uint32_t writes) {
    const int i = index++;
    if (i == drop) {
      log += std::to_string(i) + " " + name + " (left out)\n";
      return LILICORR_OK;
    }
    log += std::to_string(i) + " " + name + " reads " + names(reads) + " writes " + names(writes);
    const uint32_t missing = reads & ~written;
    if (missing) {
      log += " UNWRITTEN " + names(missing) + "\n";
      return LILICORR_EINVAL;
    }
    log += "\n";
    written |= writes;
    return LILICORR_OK;
  }
};

// The launch sequence of lilicorr_rerank over workspace `ws` (arguments
// already validated). With `audit` set nothing is launched: every step only
// records which workspace regions it reads and writes, and the audit fails at
// the first step that reads a region no earlier step has written.
int enqueue_rerank(const void* logits, int B, int V, int K, const lilicorr_params& pr, char* ws,
                   int32_t* out_tokens, Audit* audit) {
  const lilicorr_params* p = &pr;
  hipStream_t st = (hipStream_t)p->stream;
  const int N = p->num_blocks;
  const lilicorr_dims& d = p->weights->dims;
  const int H = d.hidden, F = d.ffn, de = d.d_e, heads = d.heads;
  const int rows = N * B;
  const int M = rows * K;
  const WeightPtrs W = weight_ptrs(*p->weights);
  const RerankWs L = rerank_ws_layout(N, B, V, K, d);
  const TopkWs TL = topk_ws_layout(rows, V, K);
  char* tws = ws + L.topk;
  int32_t* topk_idx = p->dbg_topk_idx ? p->dbg_topk_idx : (int32_t*)(ws + L.topk_idx);
  float* topk_logp = p->dbg_topk_logp ? p->dbg_topk_logp : (float*)(ws + L.topk_logp);
  float* x = (float*)(ws + L.x);
  uint16_t* hid = (uint16_t*)(ws + L.hid);
  uint16_t* u = (uint16_t*)(ws + L.u);
  uint16_t* qkv = (uint16_t*)(ws + L.qkv);
  uint16_t* attn = (uint16_t*)(ws + L.attn);
  float* heads_v = (float*)(ws + L.heads);
  uint16_t* outv = p->dbg_outv ? p->dbg_outv : (uint16_t*)(ws + L.outv);
  uint16_t* inv = p->dbg_inv ? p->dbg_inv : (uint16_t*)(ws + L.inv);
  float* gpart = (float*)(ws + L.gemm_part);
  // optional events around one stage (measurement only)
  const bool timing = p->timing_begin != nullptr;
  auto mark = [&](int stage, bool end) -> hipError_t {
    if (audit || !timing || stage != p->timing_stage) return hipSuccess;
    return hipEventRecord((hipEvent_t)(end ? p->timing_end : p->timing_begin), st);
  };
#define LL_STAGE(stage, ...)          \
  do {                                \
    LL_TRY(mark((stage), false));     \
    __VA_ARGS__;                      \
    LL_TRY(mark((stage), true));      \
  } while (0)
  // one launch: its workspace reads and writes (WS_* bits), then the launch
#define LL_STEP(name, reads, writes, launch)                               \
  do {                                                                     \
    if (audit) {                                                           \
      const int _a = audit->step((name), (reads), (writes));               \
      if (_a != LILICORR_OK) return _a;                                    \
    } else {                                                               \
      LL_TRY(launch);                                                      \
    }                                                                      \
  } while (0)

  const bool paper = d.target_hidden > 0;
  const int Bl = paper ? B - 1 : B;             // slots in the lattice
  const int Mp = N * Bl * K;                    // lattice rows
  auto resid_norm = [&](const float* gamma) {
    LinearEpilogue e;
    e.kind = EPI_RESID_F32;
    e.resid = x;
    e.norm_gamma = gamma;
    e.eps = kRmsEps;
    e.norm_out = u;
    return e;
  };
  auto plain = [](int kind) {
    LinearEpilogue e;
    e.kind = kind;
    return e;
  };
  // the split-K scratch of a linear is written and read inside its own launch
  const uint32_t GP = WS_BIT(GEMM_PART);
  // every row of the out / in vectors
  const uint32_t VEC_ALL = WS_BIT(OUTV) | WS_BIT(INV) | WS_BIT(OUTV_SLOT0) | WS_BIT(INV_SLOT0);

  // Lattice head with rows split into chunks (few tokens, or K = 8): the node
  // build merges the chunk outputs itself (one launch fewer).
  const int topk_P = topk_chunks_per_row(rows, V);
  const bool merge_in_node = !paper && linear_takes_node_source(M, H, H) && node_build_merges(N, B, K, H, topk_P);
  // a1: log-partition + top-K (the chunk partials are scratch of this launch)
  if (merge_in_node) {
    LL_STAGE(LILICORR_STAGE_TOPK,
             LL_STEP("topk_chunks", 0, WS_BIT(TOPK_PART),
                     launch_topk_lse(logits, rows, V, K, p->logits_dtype, (float*)(tws + TL.part_val),
                                     (int32_t*)(tws + TL.part_idx), (float*)(tws + TL.part_ms),
                                     topk_idx, topk_logp, p->dbg_lse, st, false)));
  } else {
    LL_STAGE(LILICORR_STAGE_TOPK,
             LL_STEP("topk_lse", 0, WS_BIT(TOPK_PART) | WS_BIT(TOPK_IDX) | WS_BIT(TOPK_LOGP),
                     launch_topk_lse(logits, rows, V, K, p->logits_dtype, (float*)(tws + TL.part_val),
                                     (int32_t*)(tws + TL.part_idx), (float*)(tws + TL.part_ms),
                                     topk_idx, topk_logp, p->dbg_lse, st)));
  }
  if (!paper && linear_takes_node_source(M, H, H)) {
    // a2: nodes. x = ((E + S) + R) + (W2c . hid + b2c); u = bf16(RMSNorm(x; gamma1 of layer 0)).
    // The table sum ((E + S) + R) is formed by the W2c linear's epilogue from
    // the tables (same float32 order), so x is written once.
    NodeSource nd;
    nd.tok = topk_idx;
    nd.E = W.E;
    nd.S = W.S;
    nd.R = W.R;
    nd.K = K;
    nd.B = B;
    nd.V = V;
    nd.magic_k = div_magic(K);
    nd.magic_b = div_magic(B);
    LinearEpilogue e = resid_norm(W.layer[0].gamma1);
    e.resid = nullptr;
    e.node = &nd;
    if (merge_in_node)
      LL_STAGE(LILICORR_STAGE_NODE,
               LL_STEP("node_build_merge", WS_BIT(TOPK_PART), WS_BIT(TOPK_IDX) | WS_BIT(TOPK_LOGP) | WS_BIT(HID),
                       launch_node_build_merge((float*)(tws + TL.part_val), (int32_t*)(tws + TL.part_idx),
                                               (float*)(tws + TL.part_ms), topk_P, topk_idx, topk_logp,
                                               p->dbg_lse, N, B, K, H, W.conf_w1, W.conf_b1, hid, V, st)));
    else
      LL_STAGE(LILICORR_STAGE_NODE,
               LL_STEP("node_build", WS_BIT(TOPK_IDX) | WS_BIT(TOPK_LOGP), WS_BIT(HID),
                       launch_node_build(topk_idx, topk_logp, N, B, K, H, W.E, nullptr, W.S, W.R,
                                         W.conf_w1, W.conf_b1, hid, nullptr, V, st)));
    LL_STAGE(LILICORR_STAGE_CONF_LINEAR,
             LL_STEP("linear_conf_w2", WS_BIT(HID) | WS_BIT(TOPK_IDX), WS_BIT(X) | WS_BIT(U) | GP,
                     launch_linear(hid, M, H, W.conf_w2, H, W.conf_b2, e, x, gpart, st)));
  } else if (!paper) {
    // a2 with the table sum written by the node build (few-row shapes whose
    // W2c linear has no node-source epilogue)
    LL_STAGE(LILICORR_STAGE_NODE,
             LL_STEP("node_build", WS_BIT(TOPK_IDX) | WS_BIT(TOPK_LOGP), WS_BIT(HID) | WS_BIT(X),
                     launch_node_build(topk_idx, topk_logp, N, B, K, H, W.E, nullptr, W.S, W.R,
                                       W.conf_w1, W.conf_b1, hid, x, V, st)));
    LL_STAGE(LILICORR_STAGE_CONF_LINEAR,
             LL_STEP("linear_conf_w2", WS_BIT(HID) | WS_BIT(X), WS_BIT(X) | WS_BIT(U) | GP,
                     launch_linear(hid, M, H, W.conf_w2, H, W.conf_b2, resid_norm(W.layer[0].gamma1),
                                   x, gpart, st)));
  } else {
    // a2 (paper's head): x = (((h W_hid^T + b_hid) + S) + R) + (W2c . hid + b2c), then
    // x += E_t[tok] W_emb^T + b_emb with u = bf16(RMSNorm(x; gamma1 of layer 0))
    const int Ht = d.target_hidden, Hd = d.drafter_hidden;
    float* ph = (float*)(ws + L.ph);
    uint16_t* ae = (uint16_t*)(ws + L.ae);
    LL_STAGE(LILICORR_STAGE_NODE, {
      LL_STEP("linear_hidden", 0, WS_BIT(PH) | GP,
              launch_linear(p->hidden, N * B, Hd, W.w_hid, H, W.b_hid, plain(EPI_F32), ph, gpart, st));
      LL_STEP("node_build", WS_BIT(TOPK_IDX) | WS_BIT(TOPK_LOGP) | WS_BIT(PH), WS_BIT(HID) | WS_BIT(X),
              launch_node_build(topk_idx, topk_logp, N, B, K, H, nullptr, ph, W.S, W.R, W.conf_w1,
                                W.conf_b1, hid, x, V, st));
      LL_STEP("gather_rows", WS_BIT(TOPK_IDX), WS_BIT(AE),
              launch_gather_rows(topk_idx, N, B, K, W.E_t, Ht, V, ae, st));
    });
    LinearEpilogue add_only = plain(EPI_RESID_F32);
    add_only.resid = x;
    LL_STAGE(LILICORR_STAGE_CONF_LINEAR, {
      LL_STEP("linear_conf_w2", WS_BIT(HID) | WS_BIT(X), WS_BIT(X) | GP,
              launch_linear(hid, Mp, H, W.conf_w2, H, W.conf_b2, add_only, x, gpart, st));
      LL_STEP("linear_emb", WS_BIT(AE) | WS_BIT(X), WS_BIT(X) | WS_BIT(U) | GP,
              launch_linear(ae, Mp, Ht, W.w_emb, H, W.b_emb, resid_norm(W.layer[0].gamma1), x, gpart,
                            st));
    });
  }
  // a3: two pre-norm layers; each residual GEMM also produces the next RMSNorm
  for (int l = 0; l < 2; ++l) {
    const LayerPtrs& Lw = W.layer[l];
    const float* next_gamma = l == 0 ? W.layer[1].gamma1 : W.gamma_f;
    const int s0 = 5 * l;
    LL_STAGE(LILICORR_STAGE_QKV + s0,
             LL_STEP("linear_qkv", WS_BIT(U), WS_BIT(QKV) | GP,
                     launch_linear(u, Mp, H, Lw.wqkv, 3 * H, Lw.bqkv, plain(EPI_BF16), qkv, gpart, st)));
    if (attention_o_fusable(N, Bl, K, H, heads)) {
      // few rows: the attention launch also forms the output projection's
      // per-head split-K slices, and the linear is only its ordered reduce
      LL_STAGE(LILICORR_STAGE_ATTENTION + s0,
               LL_STEP("lattice_attention_o", WS_BIT(QKV), WS_BIT(O_PART),
                       launch_attention_o(qkv, N, Bl, K, H, heads, Lw.dist, Lw.same, Lw.wo, gpart, st)));
      LL_STAGE(LILICORR_STAGE_O + s0,
               LL_STEP("linear_o_reduce", WS_BIT(O_PART) | WS_BIT(X), WS_BIT(X) | WS_BIT(U),
                       launch_splitk_reduce(heads, Mp, H, Lw.bo, resid_norm(Lw.gamma2), x, gpart, st)));
    } else {
      LL_STAGE(LILICORR_STAGE_ATTENTION + s0,
               LL_STEP("lattice_attention", WS_BIT(QKV), WS_BIT(ATTN),
                       launch_attention(qkv, N, Bl, K, H, heads, Lw.dist, Lw.same, attn, st)));
      LL_STAGE(LILICORR_STAGE_O + s0,
               LL_STEP("linear_o", WS_BIT(ATTN) | WS_BIT(X), WS_BIT(X) | WS_BIT(U) | GP,
                       launch_linear(attn, Mp, H, Lw.wo, H, Lw.bo, resid_norm(Lw.gamma2), x, gpart, st)));
    }
    LL_STAGE(LILICORR_STAGE_FFN1 + s0,
             LL_STEP("linear_ffn1", WS_BIT(U), WS_BIT(HID) | GP,
                     launch_linear(u, Mp, H, Lw.w1, F, Lw.b1, plain(EPI_SILU_BF16), hid, gpart, st)));
    LL_STAGE(LILICORR_STAGE_FFN2 + s0,
             LL_STEP("linear_ffn2", WS_BIT(HID) | WS_BIT(X), WS_BIT(X) | WS_BIT(U) | GP,
                     launch_linear(hid, Mp, F, Lw.w2, H, Lw.b2, resid_norm(next_gamma), x, gpart, st)));
  }
  // a4: out|in heads and their unit normalisation
  if (!paper) {
    LinearEpilogue e = plain(EPI_F32);
    e.heads_out = outv;
    e.heads_in = inv;
    LL_STAGE(LILICORR_STAGE_HEADS,
             LL_STEP("linear_heads", WS_BIT(U), VEC_ALL | GP,
                     launch_linear(u, M, H, W.w_heads, 2 * de, W.b_heads, e, heads_v, gpart, st)));
  } else {
    // a4 (paper's head): tb = bf16(bf16(RMSNorm(t; gamma_t)) W_tgt^T + b_tgt);
    // y = bf16(SiLU([u, tb, bf16(u tb)] W_fuse^T + b_fuse)); out|in heads of y;
    // anchor o_0 = unit(tb W_anchor^T + b_anchor) in slot 0's rows
    const int Ht = d.target_hidden;
    uint16_t* tnorm = (uint16_t*)(ws + L.tnorm);
    uint16_t* tb = (uint16_t*)(ws + L.tb);
    float* apre = (float*)(ws + L.apre);
    uint16_t* cat = qkv;     // [Mp, 3H] bf16: the layers are done with qkv
    uint16_t* y = attn;      // [Mp, H] bf16
    LinearEpilogue e = plain(EPI_F32);
    e.heads_out = outv;           // lattice row (n, s - 1, j) -> row (n, s, j)
    e.heads_in = inv;
    e.heads_group = Bl * K;
    e.heads_skip = K;
    LL_STAGE(LILICORR_STAGE_HEADS, {
      LL_STEP("rmsnorm_target", 0, WS_BIT(TNORM),
              launch_rmsnorm_bf16(p->target, N, Ht, W.gamma_t, kRmsEps, tnorm, st));
      LL_STEP("linear_target", WS_BIT(TNORM), WS_BIT(TB) | GP,
              launch_linear(tnorm, N, Ht, W.w_tgt, H, W.b_tgt, plain(EPI_BF16), tb, gpart, st));
      LL_STEP("linear_anchor", WS_BIT(TB), WS_BIT(APRE) | GP,
              launch_linear(tb, N, H, W.w_anchor, de, W.b_anchor, plain(EPI_F32), apre, gpart, st));
      LL_STEP("concat", WS_BIT(U) | WS_BIT(TB), WS_BIT(QKV),
              launch_concat(u, tb, N, Bl * K, H, cat, st));
      LL_STEP("linear_fuse", WS_BIT(QKV), WS_BIT(ATTN) | GP,
              launch_linear(cat, Mp, 3 * H, W.w_fuse, H, W.b_fuse, plain(EPI_SILU_BF16), y, gpart, st));
      LL_STEP("linear_heads", WS_BIT(ATTN), WS_BIT(OUTV) | WS_BIT(INV) | GP,
              launch_linear(y, Mp, H, W.w_heads, 2 * de, W.b_heads, e, heads_v, gpart, st));
      LL_STEP("anchor_rows", WS_BIT(APRE), WS_BIT(OUTV_SLOT0) | WS_BIT(INV_SLOT0),
              launch_anchor_rows(apre, N, B, K, de, outv, inv, st));
    });
  }
  // a5: pair scores, a6: the commit (one fused kernel: B * K <= 512 keeps the
  // block's cosines within the kernel's LDS budget). Vectors of 256 or more:
  // the pair products first, in 256-wide d_e slices over many waves (into
  // the heads buffer, which the heads are done with), then the walk adds the
  // slices.
  LL_TRY(mark(LILICORR_STAGE_SCORES_WALK, false));
  const uint32_t walk_reads = WS_BIT(TOPK_IDX) | WS_BIT(TOPK_LOGP);
  if (de >= kPairSliceMinDe) {
    LL_STEP("pair_slices", VEC_ALL, WS_BIT(HEADS),
            launch_pair_slices(outv, inv, N, B, K, de, heads_v, st));
    LL_STEP("scores_walk", walk_reads | WS_BIT(HEADS), 0,
            launch_scores_walk(nullptr, nullptr, heads_v, pair_slice_count(de), topk_idx, topk_logp,
                               N, B, K, de, commit_rule(*p), p->dbg_cos, out_tokens, p->dbg_score,
                               p->dbg_gap, st));
  } else {
    LL_STEP("scores_walk", walk_reads | VEC_ALL, 0,
            launch_scores_walk(outv, inv, nullptr, 1, topk_idx, topk_logp, N, B, K, de,
                               commit_rule(*p), p->dbg_cos, out_tokens, p->dbg_score, p->dbg_gap,
                               st));
  }
  LL_TRY(mark(LILICORR_STAGE_SCORES_WALK, true));
#undef LL_STEP
#undef LL_STAGE
  return LILICORR_OK;
}

}  // namespace

extern "C" {

const char* lilicorr_strerror(int code) {
  switch (code) {
    case LILICORR_OK: return "ok";
    case LILICORR_EINVAL: return "invalid argument";
    case LILICORR_EUNSUPPORTED: return "unsupported dtype, geometry or device (gfx950 only)";
    case LILICORR_EWORKSPACE: return "workspace missing or too small";
    case LILICORR_EWEIGHTS: return "weights do not match the requested dims/vocabulary";
    case LILICORR_EHIP: return "HIP runtime or launch error";
    case LILICORR_ETOOLARGE:
      return "problem needs more than the fixed scratch of lilicorr_rerank_noalloc";
    default: return "unknown status";
  }
}

size_t lilicorr_weights_bytes(const lilicorr_dims* dims, int V) {
  if (!dims_supported(dims) || V < 1) return 0;
  return weights_total_bytes(*dims, V);
}

int lilicorr_weights_tensor(const lilicorr_dims* dims, int V, int id, size_t* offset_bytes,
                            size_t* numel, int* dtype) {
  if (!dims_supported(dims) || V < 1) return LILICORR_EINVAL;
  auto specs = weight_specs(*dims, V);
  const TensorSpec* s = find_spec(specs, id);
  if (!s) return LILICORR_EINVAL;
  if (offset_bytes) *offset_bytes = s->offset;
  if (numel) *numel = s->numel();
  if (dtype) *dtype = s->kind == WK_BF16 ? LILICORR_BF16 : LILICORR_F32;
  return LILICORR_OK;
}

size_t lilicorr_workspace_bytes(int N, int B, int V, int K, const lilicorr_dims* dims) {
  if (!sizes_ok(N, B, V, K) || !dims_supported(dims)) return 0;
  return rerank_ws_layout(N, B, V, K, *dims).total;
}

size_t lilicorr_topk_workspace_bytes(int rows, int V, int K) {
  if (rows < 1 || K < 1 || K > LILICORR_MAX_TOPK || V < K) return 0;
  return topk_ws_layout(rows, V, K).total;
}

int lilicorr_weights_init(lilicorr_weights* w, void* stream) {
  if (!w) return LILICORR_EINVAL;
  if (w->vocab < 1) return LILICORR_EINVAL;
  if (!dims_supported(&w->dims)) return LILICORR_EUNSUPPORTED;
  if (!w->dev || ((uintptr_t)w->dev & 255)) return LILICORR_EINVAL;
  if (w->bytes < weights_total_bytes(w->dims, w->vocab)) return LILICORR_EWEIGHTS;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  auto specs = weight_specs(w->dims, w->vocab);
  for (const auto& s : specs) {
    // splitmix64 of seed ^ (t << 40): the per-tensor key (host side)
    uint64_t z = (w->seed ^ ((uint64_t)s.id << 40)) + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    const uint64_t key = z ^ (z >> 31);
    LL_TRY(launch_weights_init((char*)w->dev + s.offset, s.numel(), key, s.kind, s.scale,
                               (hipStream_t)stream));
  }
  return LILICORR_OK;
}

int lilicorr_validate(const void* logits, int B, int V, int K, const lilicorr_params* p,
                      const int32_t* out_tokens) {
  return validate_args(logits, B, V, K, p, out_tokens, true);
}

int lilicorr_rerank_noalloc(const void* logits, int B, int V, int K, const lilicorr_params* p,
                            int32_t* out_tokens) {
  const int v = validate_args(logits, B, V, K, p, out_tokens, false);
  if (v != LILICORR_OK) return v;
  if (rerank_ws_layout(p->num_blocks, B, V, K, p->weights->dims).total >
      (size_t)LILICORR_NOALLOC_SCRATCH_BYTES)
    return LILICORR_ETOOLARGE;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  void* ws = nullptr;
  const int sc = scratch_address(&ws);
  if (sc != LILICORR_OK) return sc;
  return enqueue_rerank(logits, B, V, K, *p, (char*)ws, out_tokens, nullptr);
}

}  // extern "C"

namespace {

int validate_args(const void* logits, int B, int V, int K, const lilicorr_params* p,
                  const int32_t* out_tokens, bool with_workspace) {
  if (!p || !logits || !out_tokens) return LILICORR_EINVAL;
  if (p->abi_version != LILICORR_ABI_VERSION) return LILICORR_EINVAL;
  if (!sizes_ok(p->num_blocks, B, V, K)) return LILICORR_EINVAL;
  if (p->logits_dtype != LILICORR_F32 && p->logits_dtype != LILICORR_BF16)
    return LILICORR_EUNSUPPORTED;
  if ((uintptr_t)logits & 15) return LILICORR_EINVAL;
  if (p->use_logp != 0 && p->use_logp != 1) return LILICORR_EINVAL;
  const lilicorr_weights* w = p->weights;
  if (!w) return LILICORR_EINVAL;
  if (!dims_supported(&w->dims)) return LILICORR_EUNSUPPORTED;
  if (w->vocab != V || !w->dev || ((uintptr_t)w->dev & 255) ||
      w->bytes < weights_total_bytes(w->dims, w->vocab))
    return LILICORR_EWEIGHTS;
  const size_t need = rerank_ws_layout(p->num_blocks, B, V, K, w->dims).total;
  if (with_workspace &&
      (!p->workspace || p->workspace_bytes < need || ((uintptr_t)p->workspace & 255)))
    return LILICORR_EWORKSPACE;
  if (p->rule != LILICORR_RULE_GREEDY && p->rule != LILICORR_RULE_EXACT &&
      p->rule != LILICORR_RULE_SAMPLE)
    return LILICORR_EINVAL;
  if (p->rule == LILICORR_RULE_SAMPLE && (!p->temperature || !p->uniforms)) return LILICORR_EINVAL;
  if (w->dims.target_hidden > 0) {   // the paper's head: its inputs, and a drafted slot
    if (B < 2) return LILICORR_EINVAL;
    if (!p->hidden || !p->target || ((uintptr_t)p->hidden & 15) || ((uintptr_t)p->target & 15))
      return LILICORR_EINVAL;
  }
  if ((p->timing_begin == nullptr) != (p->timing_end == nullptr)) return LILICORR_EINVAL;
  if (p->timing_begin && (p->timing_stage < 0 || p->timing_stage >= LILICORR_STAGE_COUNT))
    return LILICORR_EINVAL;
  return LILICORR_OK;
}

}  // namespace

extern "C" {

int lilicorr_rerank(const void* logits, int B, int V, int K, const lilicorr_params* p,
                    int32_t* out_tokens) {
  const int v = lilicorr_validate(logits, B, V, K, p, out_tokens);
  if (v != LILICORR_OK) return v;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  return enqueue_rerank(logits, B, V, K, *p, (char*)p->workspace, out_tokens, nullptr);
}

int lilicorr_rerank_audit(int N, int B, int V, int K, const lilicorr_dims* dims, int drop_step,
                          char* report, size_t report_bytes) {
  if (!dims || !sizes_ok(N, B, V, K)) return LILICORR_EINVAL;
  if (!dims_supported(dims)) return LILICORR_EUNSUPPORTED;
  if (dims->target_hidden > 0 && B < 2) return LILICORR_EINVAL;
  lilicorr_weights w{};
  w.dims = *dims;
  w.vocab = V;
  lilicorr_params p{};
  p.abi_version = LILICORR_ABI_VERSION;
  p.num_blocks = N;
  p.logits_dtype = LILICORR_BF16;
  p.alpha = 1.f;
  p.use_logp = 1;
  p.weights = &w;
  Audit a;
  a.drop = drop_step;
  const int st = enqueue_rerank(nullptr, B, V, K, p, nullptr, nullptr, &a);
  if (report && report_bytes > 0) {
    const size_t n = a.log.size() < report_bytes - 1 ? a.log.size() : report_bytes - 1;
    std::memcpy(report, a.log.data(), n);
    report[n] = 0;
  }
  return st;
}

int lilicorr_topk_lse(const void* logits, int rows, int V, int K, int dtype, void* workspace,
                      size_t workspace_bytes, int32_t* topk_idx, float* topk_logp, float* lse,
                      void* stream) {
  if (!logits || !topk_idx || !topk_logp) return LILICORR_EINVAL;
  if (rows < 1 || K < 1 || K > LILICORR_MAX_TOPK || V < K) return LILICORR_EINVAL;
  if ((int64_t)rows * 64 > ((int64_t)1 << 31)) return LILICORR_EINVAL;
  if (dtype != LILICORR_F32 && dtype != LILICORR_BF16) return LILICORR_EUNSUPPORTED;
  if ((uintptr_t)logits & 15) return LILICORR_EINVAL;
  const TopkWs TL = topk_ws_layout(rows, V, K);
  if (!workspace || workspace_bytes < TL.total || ((uintptr_t)workspace & 255))
    return LILICORR_EWORKSPACE;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  char* w = (char*)workspace;
  return hip_status(launch_topk_lse(logits, rows, V, K, dtype, (float*)(w + TL.part_val),
                                    (int32_t*)(w + TL.part_idx), (float*)(w + TL.part_ms),
                                    topk_idx, topk_logp, lse, (hipStream_t)stream));
}

size_t lilicorr_topk_shard_workspace_bytes(int rows, int V_shard, int K) {
  return lilicorr_topk_workspace_bytes(rows, V_shard, K);
}

int lilicorr_topk_shard(const void* logits, int rows, int V_shard, int K, int dtype, int id_offset,
                        void* workspace, size_t workspace_bytes, float* part_val,
                        int32_t* part_idx, float* part_ms, void* stream) {
  if (!logits || !part_val || !part_idx || !part_ms) return LILICORR_EINVAL;
  if (rows < 1 || K < 1 || K > LILICORR_MAX_TOPK || V_shard < K) return LILICORR_EINVAL;
  if ((int64_t)rows * 64 > ((int64_t)1 << 31)) return LILICORR_EINVAL;
  if (id_offset < 0 || (int64_t)id_offset + V_shard > (int64_t)INT32_MAX) return LILICORR_EINVAL;
  if (dtype != LILICORR_F32 && dtype != LILICORR_BF16) return LILICORR_EUNSUPPORTED;
  if ((uintptr_t)logits & 15) return LILICORR_EINVAL;
  const TopkWs TL = topk_ws_layout(rows, V_shard, K);
  if (!workspace || workspace_bytes < TL.total || ((uintptr_t)workspace & 255))
    return LILICORR_EWORKSPACE;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  char* w = (char*)workspace;
  return hip_status(launch_topk_shard(logits, rows, V_shard, K, dtype, id_offset,
                                      (float*)(w + TL.part_val), (int32_t*)(w + TL.part_idx),
                                      (float*)(w + TL.part_ms), part_val, part_idx, part_ms,
                                      (hipStream_t)stream));
}

int lilicorr_topk_merge(const float* part_val, const int32_t* part_idx, const float* part_ms, int G,
                        int rows, int K, int32_t* topk_idx, float* topk_logp, float* lse,
                        void* stream) {
  if (!part_val || !part_idx || !part_ms || !topk_idx || !topk_logp) return LILICORR_EINVAL;
  if (G < 1 || G > 64 || rows < 1 || K < 1 || K > LILICORR_MAX_TOPK) return LILICORR_EINVAL;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  return hip_status(launch_topk_merge_shards(G, rows, K, part_val, part_idx, part_ms, topk_idx,
                                             topk_logp, lse, (hipStream_t)stream));
}

int lilicorr_pair_scores(const uint16_t* outv, const uint16_t* inv, int N, int B, int K, int d_e,
                         float* cos, void* stream) {
  if (!outv || !inv || !cos) return LILICORR_EINVAL;
  if (N < 1 || B < 2 || B > LILICORR_MAX_SLOTS || K < 1 || K > LILICORR_MAX_TOPK)
    return LILICORR_EINVAL;
  if (d_e < 32 || d_e % 32) return LILICORR_EUNSUPPORTED;
  if (((uintptr_t)outv & 15) || ((uintptr_t)inv & 15)) return LILICORR_EINVAL;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  return hip_status(launch_pair_scores(outv, inv, N, B, K, d_e, cos, (hipStream_t)stream));
}

int lilicorr_greedy_walk(const int32_t* topk_idx, const float* topk_logp, const float* cos, int N,
                         int B, int K, float alpha, int use_logp, int32_t* out_tokens,
                         float* score, float* gap, void* stream) {
  if (!topk_idx || !topk_logp || !out_tokens || (B > 1 && !cos)) return LILICORR_EINVAL;
  if (N < 1 || B < 1 || B > LILICORR_MAX_SLOTS || K < 1 || K > LILICORR_MAX_TOPK)
    return LILICORR_EINVAL;
  if (use_logp != 0 && use_logp != 1) return LILICORR_EINVAL;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  if (B * K <= LILICORR_MAX_LATTICE && scores_walk_lds_bytes(B, K) <= kScoresWalkMaxLds) {
    // the commit kernel of lilicorr_rerank, fed the given cosines
    CommitRule r;
    r.kind = RULE_GREEDY;
    r.alpha = alpha;
    r.use_logp = use_logp;
    return hip_status(launch_scores_walk(nullptr, nullptr, cos, 1, topk_idx, topk_logp, N, B, K, 0,
                                         r, nullptr, out_tokens, score, gap, (hipStream_t)stream));
  }
  // lattices whose cosines exceed that kernel's LDS: one wave per block
  // scanning the cosines in global memory
  return hip_status(launch_greedy_walk(topk_idx, topk_logp, cos, N, B, K, alpha, use_logp,
                                       out_tokens, score, gap, (hipStream_t)stream));
}

int lilicorr_best_path(const int32_t* topk_idx, const float* topk_logp, const float* cos, int N,
                       int B, int K, float alpha, int use_logp, int32_t* out_tokens, float* score,
                       void* stream) {
  const int a = commit_args_ok(topk_idx, topk_logp, cos, N, B, K, use_logp, out_tokens);
  if (a != LILICORR_OK) return a;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  CommitRule r;
  r.kind = RULE_EXACT;
  r.alpha = alpha;
  r.use_logp = use_logp;
  return hip_status(launch_scores_walk(nullptr, nullptr, cos, 1, topk_idx, topk_logp, N, B, K, 0, r,
                                       nullptr, out_tokens, score, nullptr, (hipStream_t)stream));
}

int lilicorr_sample_path(const int32_t* topk_idx, const float* topk_logp, const float* cos, int N,
                         int B, int K, float alpha, int use_logp, const float* temperature,
                         const float* uniforms, int32_t* out_tokens, float* proposal, float* score,
                         void* stream) {
  const int a = commit_args_ok(topk_idx, topk_logp, cos, N, B, K, use_logp, out_tokens);
  if (a != LILICORR_OK) return a;
  if (!temperature || !uniforms) return LILICORR_EINVAL;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  CommitRule r;
  r.kind = RULE_SAMPLE;
  r.alpha = alpha;
  r.use_logp = use_logp;
  r.temperature = temperature;
  r.uniforms = uniforms;
  r.proposal = proposal;
  return hip_status(launch_scores_walk(nullptr, nullptr, cos, 1, topk_idx, topk_logp, N, B, K, 0, r,
                                       nullptr, out_tokens, score, nullptr, (hipStream_t)stream));
}

size_t lilicorr_linear_workspace_bytes(int M, int Kd, int N) {
  if (M < 1 || N < 1 || Kd < 64 || Kd % 64) return 0;
  return align256(plan_linear(M, Kd, N).part_floats * 4) + 256;
}

int lilicorr_linear(const uint16_t* A, int M, int Kd, const uint16_t* W, int N, const float* bias,
                    int epilogue, const float* resid, void* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!A || !W || !out || M < 1 || N < 1 || Kd < 64) return LILICORR_EINVAL;
  if (Kd % 64) return LILICORR_EUNSUPPORTED;
  if (epilogue < 0 || epilogue > 3) return LILICORR_EINVAL;
  if (epilogue == EPI_RESID_F32 && !resid) return LILICORR_EINVAL;
  if (((uintptr_t)A & 15) || ((uintptr_t)W & 15)) return LILICORR_EINVAL;
  const GemmPlan plan = plan_linear(M, Kd, N);
  if (workspace_bytes < lilicorr_linear_workspace_bytes(M, Kd, N) ||
      (plan.split > 1 && (!workspace || ((uintptr_t)workspace & 255))))
    return LILICORR_EWORKSPACE;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  LinearEpilogue ep;
  ep.kind = epilogue;
  ep.resid = resid;
  return hip_status(
      launch_linear(A, M, Kd, W, N, bias, ep, out, (float*)workspace, (hipStream_t)stream));
}

int lilicorr_rmsnorm(const float* x, int M, int H, const float* gamma, float eps, uint16_t* out,
                     void* stream) {
  if (!x || !gamma || !out || M < 1 || H < 64 || H > 8192) return LILICORR_EINVAL;
  if (H % 64) return LILICORR_EUNSUPPORTED;
  if (((uintptr_t)x & 15) || ((uintptr_t)gamma & 15) || ((uintptr_t)out & 7))
    return LILICORR_EINVAL;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  return hip_status(launch_rmsnorm(x, M, H, gamma, eps, out, (hipStream_t)stream));
}

int lilicorr_lattice_attention(const uint16_t* qkv, int N, int B, int K, int hidden, int heads,
                               const float* dist, const float* same, uint16_t* out, void* stream) {
  if (!qkv || !dist || !same || !out) return LILICORR_EINVAL;
  if (N < 1 || B < 1 || B > LILICORR_MAX_SLOTS || K < 1 || K > LILICORR_MAX_TOPK ||
      B * K > LILICORR_MAX_LATTICE)
    return LILICORR_EINVAL;
  if (heads < 1 || hidden % heads) return LILICORR_EUNSUPPORTED;
  const int dh = hidden / heads;
  if (dh != 32 && dh != 64 && dh != 128) return LILICORR_EUNSUPPORTED;
  if (((uintptr_t)qkv & 15) || ((uintptr_t)out & 7)) return LILICORR_EINVAL;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  return hip_status(
      launch_attention(qkv, N, B, K, hidden, heads, dist, same, out, (hipStream_t)stream));
}

int lilicorr_clock_probe(uint64_t* out, int64_t window_us, void* stream) {
  if (!out || ((uintptr_t)out & 7)) return LILICORR_EINVAL;
  if (window_us < 1 || window_us > 1000000) return LILICORR_EINVAL;
  const int dc = check_device();
  if (dc != LILICORR_OK) return dc;
  return hip_status(launch_clock_probe(out, (uint64_t)window_us * 100u, (hipStream_t)stream));
}

}  // extern "C"
