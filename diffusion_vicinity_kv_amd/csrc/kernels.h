// Host-side launchers of the gfx950 kernels (one declaration per kernel
// family).  Every launcher enqueues on `st` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dinfer {

enum class DType : int { F32 = 0, BF16 = 1 };

inline size_t dtype_size(DType t) { return t == DType::F32 ? 4 : 2; }

// Row table of one pass (a vicinity step or a full refresh).  Rows of request
// r occupy [req_row_off[r], req_row_off[r] + req_nrows[r]) and hold the
// consecutive positions starting at row_pos[req_row_off[r]].
struct PassTable {
  const int* nrows;        // [1]   rows in the pass (<= the pass's row capacity)
  const int* row_req;      // [rows] request of each row
  const int* row_pos;      // [rows] position of each row in its request
  const int* req_row_off;  // [batch]
  const int* req_nrows;    // [batch] 0 = request not in this pass
  const int* req_len;      // [batch] L_r: keys each row attends over
  const int* req_bs;       // [batch] current block start position
  const int* req_active;   // [batch] request takes part in denoise/commit
  const int* req_blk;      // [batch] index of the current block
};

// ---- GEMM: out[s][m][n] = sum over K-slice s of A[m][k] * W[n][k] ---------
// (W in the packed layout of launch_pack_linear)
struct GemmPlan {
  int kind;      // 0 = skinny (rows <= 128), 1 = fat
  int mt, nt;    // skinny: 16-row tiles; 16-column tiles per wave
  int nw;        // skinny: waves per workgroup; fat: column waves (2 or 4)
  int guard;     // skinny: 1 = A has exactly m_cap rows; 0 = A readable up to 16*mt rows
  int splits;    // K splits (partials out[s][m][n], summed by the consumer)
  int mtiles;    // skinny: row tiles of 16*mt rows per (column group, split); 1 or 2
  int grid;
  int lo;        // bf16 weights: 1 = activations as hi + lo bf16 halves, 0 = bf16 only
  int ap;        // fat, bf16 weights: 1 = A given as bf16 hi and lo planes (below)
};
GemmPlan plan_gemm(DType t, int m_cap, int N, int K, int target_wgs);
// A is fp32 (split into hi/lo bf16 halves in-kernel for bf16 weights), or
// with p.ap the two planes of that split, written by its producer: hi
// [m_cap][K] bf16 followed by lo [m_cap][K] (store_hi_lo4; the same bits the
// kernel would make), so the fat kernel stages them without converting.
hipError_t launch_gemm(const GemmPlan& p, DType t, const float* A, const void* W, float* out,
                       const int* m_dev, int m_cap, int N, int K, hipStream_t st);
// The fat kernel alone (M > 128): wn = 2 or 4 column waves (128 x 64*wn
// tiles), splits K slices (1 .. K/64 bf16, K/32 fp32) writing out[s][m][n];
// ap: A as bf16 planes (bf16 weights only).
hipError_t launch_gemm_fat(DType t, int wn, int splits, const float* A, const void* W,
                           float* out, const int* m_dev, int m_cap, int N, int K, hipStream_t st,
                           bool lo = true, bool ap = false);
// The fat gate|up projection of a SwiGLU FFN with SwiGLU in its epilogue
// (bf16, one K split, 256-column tiles): A as bf16 hi/lo planes [m_cap][K],
// W the packed [N = 2F][K] (gate rows, then up rows); writes act =
// silu(gate) * up as bf16 hi/lo planes [m_cap][F] (lo m_cap * F elements
// after hi), the form the down projection reads.  N % 256 == 0.
hipError_t launch_gemm_fat_swiglu(DType t, const float* A, const void* W, float* act,
                                  const int* m_dev, int m_cap, int N, int K, hipStream_t st,
                                  bool lo = true);
// n_mats matrices W [N][K] row-major -> the packed block layout every GEMM
// here reads (gemm_split.h: 16-row groups x one MFMA vector step per 1 KB
// block, 256-row tiles stored k-step by k-step).  N % 16 == 0, K a multiple
// of the vector step (32 bf16 / 16 fp32); P must not alias W.
hipError_t launch_pack_linear(DType t, const void* W, void* P, int n_mats, int N, int K,
                              hipStream_t st);
bool gemm_shape_ok(DType t, int N, int K);
int gemm_k_chunk(DType t);
// MoE experts: out[off_e + i] = A[row_of ? row_of[off_e + i] : off_e + i] * W_e^T for
// i < e_count[e]; Wtab [E] (device array) points at each expert's packed
// [N][K] matrix; max_rows bounds any e_count.
hipError_t launch_gemm_grouped(DType t, const float* A, const int* row_of, const int* e_count,
                               const int* e_off, int E, int max_rows, const void* const* Wtab,
                               float* out, int N, int K, hipStream_t st);

// ---- row-wise kernels ------------------------------------------------------
hipError_t launch_embed(DType t, PassTable tb, int m_cap, const int* tokens, int max_len,
                        const void* emb, int d, int V, int mask_id, float alpha, const int* smooth_id,
                        const float* smooth_p, const uint8_t* smooth_valid, int B, float* x,
                        hipStream_t st);
// x[m] += sum_s P[s][m]; a[m] = rmsnorm(x[m]) * g   (S = 0: no partials)
// aps > 0: a is written as bf16 hi and lo planes (hi [m][d], lo aps elements
// after it; store_hi_lo4) for a GEMM that reads planes, instead of fp32.
hipError_t launch_add_rmsnorm(DType t, const int* nrows, int m_cap, float* x, const float* P,
                              int S, size_t p_stride, const void* g, float eps, float* a, int d,
                              hipStream_t st, size_t aps = 0);
hipError_t launch_qkv_rope_scatter(DType t, PassTable tb, int m_cap, const float* P, int S,
                                   size_t p_stride, int d, int H, int hd, const float* rope_cs,
                                   float* q_out, void* kc, void* vt, int Lp, hipStream_t st);
hipError_t launch_swiglu(const int* nrows, int m_cap, const float* P, int S, size_t p_stride,
                         int F, float* act, hipStream_t st, size_t aps = 0);   // aps: as above
// block rows of the window -> x + sum_s P[s] -> rmsnorm * g -> out[r*B + j];
// also gathers each block row's planting (row_plant_id / row_plant_bias).
hipError_t launch_final_norm(DType t, PassTable tb, int batch, int B, const float* x,
                             const float* P, int S, size_t p_stride, const void* g, float eps,
                             float* out, int d, const int* plant_id, const float* plant_bias,
                             int max_len, int* row_plant_id, float* row_plant_bias,
                             hipStream_t st);

// ---- attention ---------------------------------------------------------------
struct AttnPlan {
  int qtw;              // 16-query tiles per wave (query block = 64 * qtw)
  int q_blocks, n_split, keys_per_split;
};
// Padded cache length Lp of K [req][head][Lp][hd] and V^T [req][head][hd][Lp].
int attn_cache_len(int max_len);
AttnPlan plan_attention(int batch, int max_rows_per_req, int max_keys, int H, int target_wgs);
// p_lo (bf16 caches): probabilities into the P V MFMA as hi + lo bf16 halves
// (default), or as bf16(p) alone.  o_aps > 0: the output o [m][H*hd] is
// written as bf16 hi and lo planes, o_aps elements apart (store_hi_lo4).
hipError_t launch_attention(DType t, const AttnPlan& p, PassTable tb, int batch, int m_cap,
                            const float* q, const void* kc, const void* vt, int H, int hd,
                            int Lp, float* o_part, float* ml_part, float* o, hipStream_t st,
                            bool p_lo = true, size_t o_aps = 0);

// ---- vocab statistics ---------------------------------------------------------
struct VocabPlan {
  int n_split, chunk;
};
VocabPlan plan_vocab(int rows, int V, int target_wgs);
size_t vocab_scratch_bytes(const VocabPlan& p, int rows);
// plant_id [rows] (-1 none) and plant_bias [rows] may be null.
hipError_t launch_vocab_stats(const VocabPlan& p, const float* logits, int rows, int V,
                              const int* plant_id, const float* plant_bias, int mask_id,
                              void* scratch, int* argmax, float* conf, float* lse, int* topk_id,
                              float* topk_p, hipStream_t st);

// LM head with the vocab statistics fused into its epilogue: the projection
// kernel reduces each (row, column tile) of its logits to a record (max, sum
// of exp, top-8) after the planting bias and MASK exclusion; the merge kernel
// combines a row's records.  Records: rec_f [rows][n_tiles][10] floats, then
// rec_i [rows][n_tiles][8] ints (vocab_record_bytes).
struct VocabEpi {
  const int* row_plant_id;   // [rows] planted id (-1 none)
  const float* row_plant_bias;
  int mask_id;
  float* logits;             // [rows][N] also stored when not null
  float* rec_f;
  int* rec_i;
  int n_tiles;               // column tiles of the plan (gemm_lmhead_tiles)
};
int gemm_lmhead_tiles(const GemmPlan& p, int N);
hipError_t launch_gemm_lmhead(const GemmPlan& p, DType t, const float* A, const void* W,
                              const int* m_dev, int m_cap, int N, int K, const VocabEpi& e,
                              hipStream_t st);
hipError_t launch_gemm_fat_lmhead(DType t, int wn, const float* A, const void* W,
                                  const int* m_dev, int m_cap, int N, int K, const VocabEpi& e,
                                  hipStream_t st);
size_t vocab_record_bytes(int rows, int n_tiles);
hipError_t launch_vocab_merge_tiles(int rows, int n_tiles, const float* rec_f, const int* rec_i,
                                    int* argmax, float* conf, float* lse, int* topk_id,
                                    float* topk_p, hipStream_t st);

// ---- mixture of experts -------------------------------------------------------
hipError_t launch_moe_route(DType t, PassTable tb, int m_cap, const float* f, int d,
                            const void* Wr, int E, int top_k, const float* router_bias,
                            int n_layers, int n_blocks, int layer, int* sel, float* gate,
                            float* rlog, hipStream_t st);
hipError_t launch_moe_plan(const int* nrows, int m_cap, const int* sel, int E, int top_k,
                           int* e_count, int* e_off, int* row_of, int* pos, int* n_assign,
                           hipStream_t st);
// Expert-cache accounting of one routed layer: per expert, its assignment
// count is added to counts[e] (usage since the last placement); the
// experts with rows and their rows are split into hits (resident[e] != 0)
// and misses, added to acct[0..3] = expert hits, expert misses, row hits,
// row misses (int64).
hipError_t launch_expert_usage(const int* e_count, int E, const int* resident, int* counts,
                               long long* acct, hipStream_t st);
hipError_t launch_moe_combine(const int* nrows, int m_cap, float* x, const float* P, int S,
                              size_t p_stride, const float* Y, const int* pos, const float* gate,
                              int top_k, int d, hipStream_t st);

// ---- decode state ---------------------------------------------------------------
// Per-request decode accounting words: [0] threshold commits, [1] credit-only
// commits, [2] fallback commits, [3] idle steps (block already done), [4 + k]
// steps that committed k tokens (k = 0..64).
constexpr int kDecodeStatWords = 72;
struct CommitArgs {
  int batch, B, max_len, mask_id, hierarchical;
  int eos_id;            // -1: none
  float tau, kappa, gamma, lambda;
  const int* req_bs;
  const int* req_active;
  const int* req_len;    // L_r
  const int* req_blk;    // current block index (response start = bs - blk * B)
  int* tokens;
  const int* argmax;
  const float* conf;
  const int* topk_id;
  const float* topk_p;
  float* credit;
  int* tracked;
  int* smooth_id;
  float* smooth_p;
  uint8_t* smooth_valid;
  uint8_t* commit_mask;
  int* block_done;
  int* step_count;
  int* commit_count;
  int* decode_stats;     // [batch][kDecodeStatWords]
};
hipError_t launch_commit(const CommitArgs& a, hipStream_t st);
hipError_t launch_step_gate(int batch, int* nrows, int* lm_rows, int* req_nrows,
                            const int* req_active, const int* block_done, hipStream_t st);
hipError_t launch_block_reset(int batch, int B, const int* req_mask, float* credit, int* tracked,
                              uint8_t* smooth_valid, uint8_t* commit_mask, int* block_done,
                              int* step_count, hipStream_t st);

}  // namespace dinfer
