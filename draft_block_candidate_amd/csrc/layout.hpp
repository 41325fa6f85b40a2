// Host-side layout of the weight blob and of the rerank workspace.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <cmath>
#include <vector>

#include "kernels.hpp"
#include "lilicorr.h"

namespace ll {

enum WeightKind { WK_BF16 = 0, WK_F32 = 1, WK_GAMMA = 2 };

struct TensorSpec {
  int id;
  int64_t rows, cols;
  int kind;
  float scale;  // U(-scale, scale); unused for gains
  size_t offset;
  size_t numel() const { return (size_t)(rows * cols); }
  size_t bytes() const { return numel() * (kind == WK_BF16 ? 2 : 4); }
};

constexpr int kTableRows = 64;   // slot and rank tables
constexpr int kDistSpan = 127;   // signed slot distance -63..63

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline float inv_sqrt_scale(int fan_in) { return (float)(1.0 / std::sqrt((double)fan_in)); }

// Tensor ids, shapes and scales of the synthetic encoder (documented with
// lilicorr_weights_tensor in lilicorr.h). Offsets are 256-byte aligned and
// follow the id order.
inline std::vector<TensorSpec> weight_specs(const lilicorr_dims& d, int V) {
  const int64_t H = d.hidden, F = d.ffn, h = d.heads, de = d.d_e;
  std::vector<TensorSpec> t;
  auto add = [&](int id, int64_t r, int64_t c, int kind, float scale) {
    t.push_back(TensorSpec{id, r, c, kind, scale, 0});
  };
  const bool paper = d.target_hidden > 0;
  if (!paper) add(0, V, H, WK_BF16, 1.0f);
  add(1, kTableRows, H, WK_BF16, 1.0f);
  add(2, kTableRows, H, WK_BF16, 1.0f);
  add(3, H, 5, WK_BF16, inv_sqrt_scale(5));
  add(4, 1, H, WK_F32, inv_sqrt_scale(5));
  add(5, H, H, WK_BF16, inv_sqrt_scale((int)H));
  add(6, 1, H, WK_F32, inv_sqrt_scale((int)H));
  for (int l = 0; l < d.layers; ++l) {
    const int b = 16 + 16 * l;
    add(b + 0, 1, H, WK_GAMMA, 0.f);
    add(b + 1, 3 * H, H, WK_BF16, inv_sqrt_scale((int)H));
    add(b + 2, 1, 3 * H, WK_F32, inv_sqrt_scale((int)H));
    add(b + 3, H, H, WK_BF16, inv_sqrt_scale((int)H));
    add(b + 4, 1, H, WK_F32, inv_sqrt_scale((int)H));
    add(b + 5, 1, H, WK_GAMMA, 0.f);
    add(b + 6, F, H, WK_BF16, inv_sqrt_scale((int)H));
    add(b + 7, 1, F, WK_F32, inv_sqrt_scale((int)H));
    add(b + 8, H, F, WK_BF16, inv_sqrt_scale((int)F));
    add(b + 9, 1, H, WK_F32, inv_sqrt_scale((int)F));
    add(b + 10, h, kDistSpan, WK_F32, 0.5f);
    add(b + 11, 1, h, WK_F32, 0.5f);
  }
  add(48, 1, H, WK_GAMMA, 0.f);
  // w_out and w_in are adjacent (and so are their biases) so that one GEMM
  // with N = 2 d_e produces both heads.
  add(49, de, H, WK_BF16, inv_sqrt_scale((int)H));
  add(51, de, H, WK_BF16, inv_sqrt_scale((int)H));
  add(50, 1, de, WK_F32, inv_sqrt_scale((int)H));
  add(52, 1, de, WK_F32, inv_sqrt_scale((int)H));
  if (paper) {
    const int64_t Ht = d.target_hidden, Hd = d.drafter_hidden;
    add(56, V, Ht, WK_BF16, 1.0f);
    add(57, H, Ht, WK_BF16, inv_sqrt_scale((int)Ht));
    add(58, 1, H, WK_F32, inv_sqrt_scale((int)Ht));
    add(59, H, Hd, WK_BF16, inv_sqrt_scale((int)Hd));
    add(60, 1, H, WK_F32, inv_sqrt_scale((int)Hd));
    add(61, 1, Ht, WK_GAMMA, 0.f);
    add(62, H, Ht, WK_BF16, inv_sqrt_scale((int)Ht));
    add(63, 1, H, WK_F32, inv_sqrt_scale((int)Ht));
    add(64, H, 3 * H, WK_BF16, inv_sqrt_scale((int)(3 * H)));
    add(65, 1, H, WK_F32, inv_sqrt_scale((int)(3 * H)));
    add(66, de, H, WK_BF16, inv_sqrt_scale((int)H));
    add(67, 1, de, WK_F32, inv_sqrt_scale((int)H));
  }
  size_t off = 0;
  for (auto& s : t) {
    // w_in directly follows w_out, b_in directly follows b_out
    if (s.id == 51 || s.id == 52) {
      s.offset = off;
    } else {
      off = align256(off);
      s.offset = off;
    }
    off += s.bytes();
  }
  return t;
}

inline size_t weights_total_bytes(const lilicorr_dims& d, int V) {
  auto t = weight_specs(d, V);
  const auto& last = t.back();
  return align256(last.offset + last.bytes());
}

inline const TensorSpec* find_spec(const std::vector<TensorSpec>& t, int id) {
  for (const auto& s : t)
    if (s.id == id) return &s;
  return nullptr;
}

// Device pointers into an initialised blob.
struct LayerPtrs {
  const float *gamma1, *bqkv, *bo, *gamma2, *b1, *b2, *dist, *same;
  const uint16_t *wqkv, *wo, *w1, *w2;
};

struct WeightPtrs {
  const uint16_t *E, *S, *R, *conf_w1, *conf_w2, *w_heads;
  const float *conf_b1, *conf_b2, *gamma_f, *b_heads;
  LayerPtrs layer[2];
  // the paper's head (null for the lattice head)
  const uint16_t *E_t, *w_emb, *w_hid, *w_tgt, *w_fuse, *w_anchor;
  const float *b_emb, *b_hid, *gamma_t, *b_tgt, *b_fuse, *b_anchor;
};

inline WeightPtrs weight_ptrs(const lilicorr_weights& w) {
  auto t = weight_specs(w.dims, w.vocab);
  const char* base = (const char*)w.dev;
  auto P = [&](int id) -> const void* {
    const TensorSpec* sp = find_spec(t, id);
    return sp ? base + sp->offset : nullptr;
  };
  WeightPtrs p;
  p.E = (const uint16_t*)P(0);
  p.S = (const uint16_t*)P(1);
  p.R = (const uint16_t*)P(2);
  p.conf_w1 = (const uint16_t*)P(3);
  p.conf_b1 = (const float*)P(4);
  p.conf_w2 = (const uint16_t*)P(5);
  p.conf_b2 = (const float*)P(6);
  for (int l = 0; l < 2; ++l) {
    const int b = 16 + 16 * l;
    LayerPtrs& L = p.layer[l];
    L.gamma1 = (const float*)P(b + 0);
    L.wqkv = (const uint16_t*)P(b + 1);
    L.bqkv = (const float*)P(b + 2);
    L.wo = (const uint16_t*)P(b + 3);
    L.bo = (const float*)P(b + 4);
    L.gamma2 = (const float*)P(b + 5);
    L.w1 = (const uint16_t*)P(b + 6);
    L.b1 = (const float*)P(b + 7);
    L.w2 = (const uint16_t*)P(b + 8);
    L.b2 = (const float*)P(b + 9);
    L.dist = (const float*)P(b + 10);
    L.same = (const float*)P(b + 11);
  }
  p.gamma_f = (const float*)P(48);
  p.w_heads = (const uint16_t*)P(49);
  p.b_heads = (const float*)P(50);
  p.E_t = (const uint16_t*)P(56);
  p.w_emb = (const uint16_t*)P(57);
  p.b_emb = (const float*)P(58);
  p.w_hid = (const uint16_t*)P(59);
  p.b_hid = (const float*)P(60);
  p.gamma_t = (const float*)P(61);
  p.w_tgt = (const uint16_t*)P(62);
  p.b_tgt = (const float*)P(63);
  p.w_fuse = (const uint16_t*)P(64);
  p.b_fuse = (const float*)P(65);
  p.w_anchor = (const uint16_t*)P(66);
  p.b_anchor = (const float*)P(67);
  return p;
}

// ---- top-K work split ----------------------------------------------------
// One wave streams one contiguous chunk of a row. Rows are split into enough
// chunks to give the GPU about kTopkTargetWaves waves, each chunk at least
// kTopkMinChunk elements, and at most 64 chunks per row (the merge assigns one
// lane per chunk).
#ifndef LL_TOPK_TARGET_WAVES
#define LL_TOPK_TARGET_WAVES 4096
#endif
constexpr int kTopkTargetWaves = LL_TOPK_TARGET_WAVES;
constexpr int64_t kTopkMinChunk = 2048;

inline int topk_chunks_per_row(int rows, int V) {
  int64_t want = (kTopkTargetWaves + rows - 1) / rows;
  int64_t max_by_len = (V + kTopkMinChunk - 1) / kTopkMinChunk;
  int64_t c = want < max_by_len ? want : max_by_len;
  if (c < 1) c = 1;
  if (c > 64) c = 64;
  return (int)c;
}

struct TopkWs {
  size_t part_val, part_idx, part_ms, total;
};

inline TopkWs topk_ws_layout(int rows, int V, int K) {
  const size_t P = (size_t)topk_chunks_per_row(rows, V);
  TopkWs w;
  size_t off = 0;
  w.part_val = off;
  off = align256(off + (size_t)rows * P * K * 4);
  w.part_idx = off;
  off = align256(off + (size_t)rows * P * K * 4);
  w.part_ms = off;
  off = align256(off + (size_t)rows * P * 8);
  w.total = off;
  return w;
}

// ---- rerank workspace ------------------------------------------------------
struct RerankWs {
  size_t topk, topk_idx, topk_logp, x, hid, u, qkv, attn, heads, outv, inv, gemm_part;
  // the paper's head: projected hidden states [N B, H] f32, gathered target
  // embedding rows [M', H_t] bf16, normalised target [N, H_t] bf16, projected
  // target [N, H] bf16, anchor head before normalisation [N, d_e] f32
  // (M' = N (B-1) K)
  size_t ph, ae, tnorm, tb, apre;
  size_t total;
};

// Largest split-K scratch over the linear layers of one rerank call (M rows
// of the lattice; the paper's head adds products over N B and N rows).
inline size_t rerank_gemm_scratch(int M, const lilicorr_dims& d, int NB = 0, int N = 0) {
  const int H = d.hidden, F = d.ffn, de = d.d_e, Ht = d.target_hidden, Hd = d.drafter_hidden;
  const int shapes[6][2] = {{H, H}, {H, 3 * H}, {H, H}, {H, F}, {F, H}, {H, 2 * de}};  // (Kd, N)
  size_t pf = 0;
  for (const auto& sh : shapes) {
    const GemmPlan p = plan_linear(M, sh[0], sh[1]);
    if (p.part_floats > pf) pf = p.part_floats;
  }
  if (Ht > 0) {
    const int more[5][3] = {{M, Ht, H}, {M, 3 * H, H}, {NB, Hd, H}, {N, Ht, H}, {N, H, de}};  // (M, Kd, N)
    for (const auto& sh : more) {
      const GemmPlan p = plan_linear(sh[0], sh[1], sh[2]);
      if (p.part_floats > pf) pf = p.part_floats;
    }
  }
  return pf;
}

inline RerankWs rerank_ws_layout(int N, int B, int V, int K, const lilicorr_dims& d) {
  const size_t rows = (size_t)N * B;
  const size_t M = rows * K;
  const size_t H = d.hidden, F = d.ffn, de = d.d_e;
  RerankWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  w.topk = take(topk_ws_layout((int)rows, V, K).total);
  w.topk_idx = take(rows * K * 4);
  w.topk_logp = take(rows * K * 4);
  w.x = take(M * H * 4);
  w.hid = take(M * (F > H ? F : H) * 2);
  w.u = take(M * H * 2);
  w.qkv = take(M * 3 * H * 2);
  w.attn = take(M * H * 2);
  w.heads = take(M * 2 * de * 4);
  w.outv = take(M * de * 2);
  w.inv = take(M * de * 2);
  const bool paper = d.target_hidden > 0;
  const size_t Mp = paper ? (size_t)N * (B - 1) * K : M;   // lattice rows
  size_t pf = rerank_gemm_scratch((int)Mp, d, N * B, N);
  // attention fused with the output projection's per-head K slices
  if (attention_o_fusable(N, paper ? B - 1 : B, K, (int)H, d.heads) && (size_t)d.heads * Mp * H > pf)
    pf = (size_t)d.heads * Mp * H;
  w.gemm_part = take(pf * 4);
  w.ph = w.ae = w.tnorm = w.tb = w.apre = 0;
  if (paper) {
    const size_t Ht = d.target_hidden;
    w.ph = take(rows * H * 4);
    w.ae = take(Mp * Ht * 2);
    w.tnorm = take((size_t)N * Ht * 2);
    w.tb = take((size_t)N * H * 2);
    w.apre = take((size_t)N * de * 4);
  }
  w.total = off;
  return w;
}

}  // namespace ll
