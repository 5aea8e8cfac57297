// Host runtime behind the C ABI of include/dinfer.h: configuration checks,
// workspace carve-up, per-pass row tables, the launch sequence of a refresh
// and of a denoising step, block bookkeeping, and HIP-graph replay of several
// steps per host wait (dInfer news article, section "系统级压榨": loop
// unrolling removes the bubbles between iterations; dLLM-serving
// characterisation, "GPU vs. CPU overhead": CPU dispatch dominates a
// single request's wall time).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/dinfer.h"
#include "kernels.h"

using namespace dinfer;

namespace {

thread_local std::string g_last_error;

dinfer_status fail(dinfer_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(DINFER_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));     \
  } while (0)

constexpr size_t kAlign = 256;

// Scratch of dinfer_vocab_stats_noalloc: the split partials of the vocab
// statistics live in this fixed device array instead of a caller buffer.
// Each GPU the library runs on holds its own copy until the process ends.
constexpr size_t kNoAllocScratchBytes = size_t(2) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
// Device address of `scratch` per device, looked up once (with that device
// current) by hipGetSymbolAddress; host code passes only these addresses to
// kernels, never the array's name.
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
constexpr int64_t kSchedMaxBudget = int64_t(1) << 62;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Row capacities and buffer sizes derived from the configuration.
struct Layout {
  int d, H, hd, F, V, nl, B, w;
  int max_batch, max_len;
  int Lp;                       // cache length per head row (max_len padded to 64)
  int m_step, m_ref, m_all;     // row capacities: step pass, refresh pass, either
  int lm_rows;                  // max_batch * B
  DType dt;
  GemmPlan g_qkv_s, g_o_s, g_gu_s, g_d_s, g_lm;   // step pass
  GemmPlan g_qkv_r, g_o_r, g_gu_r, g_d_r;         // refresh pass
  // MoE: the shared expert reuses the FFN plans (sized for Fs); the experts
  // use the grouped GEMM
  bool moe;
  int E, topk, Fe, Fs, assign_cap;
  AttnPlan a_step, a_ref;
  int lm_tiles;                 // column tiles of the LM head (vocab records per row)
  size_t part_elems, attn_o_elems, attn_ml_elems;
  // byte offsets
  size_t off_rope, off_kvk, off_kvv, off_x, off_a, off_q, off_o, off_act, off_part, off_ao,
      off_aml, off_hf, off_logits, off_lmrec, off_rpid, off_rpb, off_argmax, off_conf, off_lse,
      off_tid, off_tp, off_credit, off_tracked, off_sid, off_sp, off_sv, off_cm, off_done,
      off_steps, off_ccount, off_dstat, off_tab_step, off_tab_ref, off_mask, off_misc, off_sel, off_gate,
      off_pos, off_rowof, off_ecount, off_eoff, off_nassign, off_egu, off_eact, off_ey, off_rlog,
      off_wtab, off_resident, off_eusage, off_eacct,
      total;
  size_t kv_layer_elems;        // elements of one layer's K (or V) cache
  int tab_ints_step, tab_ints_ref;
};

int table_ints(int m_cap, int mb) { return 16 + 2 * m_cap + 7 * mb; }

bool make_layout(const dinfer_model_cfg* m, const dinfer_decode_cfg* dc, int max_batch,
                 int max_len, Layout* L, std::string* why) {
  auto bad = [&](const char* s) {
    if (why) *why = s;
    return false;
  };
  if (!m || !dc) return bad("null config");
  if (m->dtype != DINFER_F32 && m->dtype != DINFER_BF16) return bad("dtype must be F32 or BF16");
  if (m->n_layers < 1 || m->d_model < 1 || m->n_heads < 1 || m->head_dim < 1 || m->vocab < 2)
    return bad("model dimensions must be positive");
  if (m->n_heads * m->head_dim != m->d_model) return bad("n_heads * head_dim must equal d_model");
  if (m->head_dim != 64 && m->head_dim != 128) return bad("head_dim must be 64 or 128");
  if (m->mask_id < 0 || m->mask_id >= m->vocab) return bad("mask_id out of range");
  const bool moe = m->n_experts > 0;
  if (moe) {
    if (m->top_k < 1 || m->top_k > m->n_experts) return bad("top_k must be in 1..n_experts");
    if (m->n_experts > 64) return bad("n_experts above 64 is not supported");
    if (m->top_k > 8) return bad("top_k above 8 is not supported");
    if (m->expert_ffn < 1 || m->shared_ffn < 1) return bad("expert_ffn and shared_ffn must be positive");
    // the router's lanes walk d in 16-byte steps, 64 lanes at a time
    if (m->d_model % (m->dtype == DINFER_BF16 ? 512 : 256) != 0)
      return bad("MoE d_model must be a multiple of 512 (bf16) or 256 (f32)");
  } else if (m->ffn_dim < 1) {
    return bad("ffn_dim must be positive");
  }
  if (m->d_model > 8192) return bad("d_model above 8192");
  if (m->vocab % 4 != 0) return bad("vocab must be a multiple of 4");
  if (dc->block_len < 1 || dc->block_len > 64) return bad("block_len must be in 1..64");
  if (dc->vicinity_w < 0) return bad("vicinity_w must be >= 0");
  if (dc->smooth_topk != 8) return bad("smooth_topk must be 8");
  if (dc->graph_unroll < 0 || dc->graph_unroll > 64) return bad("graph_unroll must be in 0..64");
  if (dc->eos_id != -1 && (dc->eos_id < 0 || dc->eos_id >= m->vocab || dc->eos_id == m->mask_id))
    return bad("eos_id must be -1 or a token id in [0, vocab) other than mask_id");
  if (max_batch < 1 || max_len < 1) return bad("max_batch and max_len must be positive");
  const DType dt = m->dtype == DINFER_F32 ? DType::F32 : DType::BF16;
  const int d = m->d_model, F = m->ffn_dim, V = m->vocab;
  const int Fe = m->expert_ffn, Fs = m->shared_ffn;
  bool shapes = gemm_shape_ok(dt, 3 * d, d) && gemm_shape_ok(dt, d, d) && gemm_shape_ok(dt, V, d);
  if (moe)
    shapes = shapes && gemm_shape_ok(dt, 2 * Fe, d) && gemm_shape_ok(dt, d, Fe) &&
             gemm_shape_ok(dt, 2 * Fs, d) && gemm_shape_ok(dt, d, Fs);
  else
    shapes = shapes && gemm_shape_ok(dt, 2 * F, d) && gemm_shape_ok(dt, d, F);
  if (!shapes) return bad("GEMM shapes must have N % 128 == 0 and K % 128 (bf16) / 64 (f32) == 0");

  Layout& l = *L;
  l.dt = dt;
  l.d = d;
  l.H = m->n_heads;
  l.hd = m->head_dim;
  l.F = F;
  l.V = V;
  l.nl = m->n_layers;
  l.B = dc->block_len;
  l.w = dc->vicinity_w;
  l.max_batch = max_batch;
  l.max_len = max_len;
  const int win = std::min(max_len, l.B + 2 * l.w);
  l.m_step = max_batch * win;
  l.m_ref = max_batch * max_len;
  l.m_all = (std::max(l.m_step, l.m_ref) + 15) / 16 * 16;   // 16-row padded buffers
  l.lm_rows = max_batch * l.B;
  l.moe = moe;
  l.E = m->n_experts;
  l.topk = moe ? m->top_k : 0;
  l.Fe = Fe;
  l.Fs = Fs;
  const int tw = 256;   // about one skinny workgroup per CU
  const int Fd = moe ? Fs : F;   // the dense FFN, or the shared expert
  l.g_qkv_s = plan_gemm(dt, l.m_step, 3 * d, d, tw);
  l.g_o_s = plan_gemm(dt, l.m_step, d, d, tw);
  l.g_gu_s = plan_gemm(dt, l.m_step, 2 * Fd, d, tw);
  l.g_d_s = plan_gemm(dt, l.m_step, d, Fd, tw);
  l.g_lm = plan_gemm(dt, l.lm_rows, V, d, tw);
  // the logits are read in place by the vocab statistics: one K slice only
  if (l.g_lm.splits != 1) {
    l.g_lm.grid /= l.g_lm.splits;
    l.g_lm.splits = 1;
  }
  // the step's activation buffers hold at least 16*mt rows: no row guards,
  // except where two row tiles read past the step's rows
  for (GemmPlan* g : {&l.g_qkv_s, &l.g_o_s, &l.g_gu_s, &l.g_d_s, &l.g_lm})
    g->guard = g->kind == 0 && g->mtiles > 1 && l.m_step < 16 * g->mt * g->mtiles;
  l.g_qkv_r = plan_gemm(dt, l.m_ref, 3 * d, d, tw);
  l.g_o_r = plan_gemm(dt, l.m_ref, d, d, tw);
  l.g_gu_r = plan_gemm(dt, l.m_ref, 2 * Fd, d, tw);
  l.g_d_r = plan_gemm(dt, l.m_ref, d, Fd, tw);
  for (GemmPlan* g : {&l.g_qkv_r, &l.g_o_r, &l.g_gu_r, &l.g_d_r}) g->guard = 0;
  auto pe = [](const GemmPlan& g, int m_cap, int N) { return (size_t)g.splits * m_cap * N; };
  l.part_elems = std::max({pe(l.g_qkv_s, l.m_step, 3 * d), pe(l.g_o_s, l.m_step, d),
                           pe(l.g_gu_s, l.m_step, 2 * Fd), pe(l.g_d_s, l.m_step, d),
                           pe(l.g_qkv_r, l.m_ref, 3 * d), pe(l.g_o_r, l.m_ref, d),
                           pe(l.g_gu_r, l.m_ref, 2 * Fd), pe(l.g_d_r, l.m_ref, d)});
  // about one workgroup per CU: more key splits only add fp32 partial traffic
  l.a_step = plan_attention(max_batch, win, max_len, l.H, 256);
  l.a_ref = plan_attention(max_batch, max_len, max_len, l.H, 256);
  l.attn_o_elems = std::max((size_t)l.a_step.n_split * l.m_step, (size_t)l.a_ref.n_split * l.m_ref) *
                   l.H * l.hd;
  l.attn_ml_elems = l.attn_o_elems / l.hd * 2;
  l.lm_tiles = gemm_lmhead_tiles(l.g_lm, V);
  l.tab_ints_step = table_ints(l.m_step, max_batch);
  l.tab_ints_ref = table_ints(l.m_ref, max_batch);
  l.Lp = attn_cache_len(max_len);
  l.kv_layer_elems = (size_t)max_batch * l.H * l.Lp * l.hd;

  const size_t es = dtype_size(dt);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  l.off_rope = take((size_t)max_len * l.hd * 4);
  l.off_kvk = take(l.kv_layer_elems * l.nl * es);
  l.off_kvv = take(l.kv_layer_elems * l.nl * es);
  l.off_x = take((size_t)l.m_all * d * 4);
  l.off_a = take((size_t)l.m_all * d * 4);
  l.off_q = take((size_t)l.m_all * d * 4);
  l.off_o = take((size_t)l.m_all * d * 4);
  l.off_act = take((size_t)l.m_all * Fd * 4);
  l.off_part = take(l.part_elems * 4);
  l.off_ao = take(l.attn_o_elems * 4);
  l.off_aml = take(l.attn_ml_elems * 4);
  l.off_hf = take((size_t)(l.lm_rows + 15) / 16 * 16 * d * 4);
  l.off_logits = take((size_t)l.lm_rows * V * 4);
  l.off_lmrec = take(vocab_record_bytes(l.lm_rows, l.lm_tiles));
  l.off_rpid = take((size_t)l.lm_rows * 4);
  l.off_rpb = take((size_t)l.lm_rows * 4);
  l.off_argmax = take((size_t)l.lm_rows * 4);
  l.off_conf = take((size_t)l.lm_rows * 4);
  l.off_lse = take((size_t)l.lm_rows * 4);
  l.off_tid = take((size_t)l.lm_rows * 8 * 4);
  l.off_tp = take((size_t)l.lm_rows * 8 * 4);
  l.off_credit = take((size_t)l.lm_rows * 4);
  l.off_tracked = take((size_t)l.lm_rows * 4);
  l.off_sid = take((size_t)l.lm_rows * 8 * 4);
  l.off_sp = take((size_t)l.lm_rows * 8 * 4);
  l.off_sv = take((size_t)l.lm_rows);
  l.off_cm = take((size_t)l.lm_rows);
  l.off_done = take((size_t)max_batch * 4);
  l.off_steps = take((size_t)max_batch * 4);
  l.off_ccount = take((size_t)max_batch * 4);
  l.off_dstat = take((size_t)max_batch * kDecodeStatWords * 4);
  l.off_tab_step = take((size_t)l.tab_ints_step * 4);
  l.off_tab_ref = take((size_t)l.tab_ints_ref * 4);
  l.off_mask = take((size_t)max_batch * 4);
  l.off_misc = take(64);
  l.assign_cap = l.m_all * l.topk;
  const size_t ac = moe ? (size_t)l.assign_cap : 0;
  l.off_sel = take(ac * 4);
  l.off_gate = take(ac * 4);
  l.off_pos = take(ac * 4);
  l.off_rowof = take(ac * 4);
  l.off_ecount = take((size_t)(moe ? l.E : 0) * 4);
  l.off_eoff = take((size_t)(moe ? l.E : 0) * 4);
  l.off_nassign = take(64);
  l.off_egu = take(ac * 2 * Fe * 4);
  l.off_eact = take(ac * Fe * 4);
  l.off_ey = take(ac * d * 4);
  l.off_rlog = take((size_t)(moe ? l.m_all * l.E : 0) * 4);
  // MoE expert pointer tables [layer][gate|up, down][E], residency flags,
  // usage counts since the last placement [layer][E], accounting [layer][4]
  const size_t ne = moe ? (size_t)l.nl * l.E : 0;
  l.off_wtab = take(ne * 2 * sizeof(void*));
  l.off_resident = take(ne * 4);
  l.off_eusage = take(ne * 4);
  l.off_eacct = take((moe ? (size_t)l.nl : 0) * 4 * 8);
  l.total = o;
  return true;
}

PassTable table_view(int* base, int m_cap, int mb) {
  PassTable t;
  t.nrows = base;
  t.row_req = base + 16;
  t.row_pos = base + 16 + m_cap;
  t.req_row_off = base + 16 + 2 * m_cap;
  t.req_nrows = t.req_row_off + mb;
  t.req_len = t.req_nrows + mb;
  t.req_bs = t.req_len + mb;
  t.req_active = t.req_bs + mb;
  t.req_blk = t.req_active + mb;
  return t;
}

}  // namespace

struct dinfer_ctx {
  dinfer_model_cfg m;
  dinfer_decode_cfg dc;
  Layout L;
  // refresh pass: row capacity and projection plans for the rows of the
  // current refresh call (the table keeps the full m_ref layout)
  int ref_mcap = 0;
  GemmPlan ref_q{}, ref_o{}, ref_g{}, ref_d{};
  hipStream_t stream = nullptr;   // caller's stream
  hipStream_t st = nullptr;       // stream kernels go to (the capture stream while capturing)
  hipStream_t cap_stream = nullptr;
  // MoE: the shared expert runs on a second stream beside the routed
  // experts (forked and joined with events, in eager passes and in the
  // captured step graph alike)
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // weights
  const void* tok_emb = nullptr;
  const void* final_norm = nullptr;
  const void* lm_head = nullptr;
  std::vector<const void*> attn_norm, wqkv, wo, ffn_norm, wgu, wd;
  std::vector<const void*> router, egu, ed, sgu, sd;   // MoE
  // workspace
  char* ws = nullptr;
  // batch
  int batch = 0;
  int* tokens = nullptr;
  const int* plant_id = nullptr;
  const float* plant_bias = nullptr;
  const float* router_bias = nullptr;
  int n_bias_blocks = 0;                 // blocks per request in the router bias array
  std::vector<int> P, G, Lr, blk, nblk;
  std::vector<uint8_t> finished, refreshed;
  // host staging (pinned) for the row tables
  int* h_tab_step = nullptr;
  int* h_tab_ref = nullptr;
  int* h_misc = nullptr;
  // MoE expert tables (host staging, pinned) and the expert cache
  const void** h_wtab = nullptr;      // [layer][2][E]
  int* h_resident = nullptr;          // [layer][E]
  bool experts_ready = false;         // every table entry points at weights
  bool offload = false;
  int slots = 0, interval = 0;
  char* d_slots = nullptr;
  std::vector<const char*> h_gu, h_dn;       // host store, host addresses
  std::vector<const char*> hd_gu, hd_dn;     // the same, device-accessible
  std::vector<std::vector<int>> slot_expert; // [layer][slot] -> expert
  long long bytes_h2d = 0, placements = 0;
  int steps_since_place = 0;
  hipEvent_t ev_step_upload = nullptr, ev_ref_upload = nullptr;
  bool step_dirty = true;
  int state = 0;                  // 0 init, 1 batch bound
  bool stats_ready = false;
  bool keep_logits = false;       // the LM head also stores the fp32 logits
  // projections whose activations enter the MFMA in bf16 only (bit 0 QKV,
  // 1 O, 2 gate|up, 3 down), in steps and in refreshes; 0 = hi + lo everywhere
  uint32_t hi_only_step = 0, hi_only_refresh = 0;
  // graph
  hipGraphExec_t graph = nullptr;
  int graph_steps = 0;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;

  template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
};

namespace {

dinfer_status upload_step_table(dinfer_ctx* c) {
  const Layout& L = c->L;
  HIP_TRY(hipEventSynchronize(c->ev_step_upload));
  int* t = c->h_tab_step;
  const int mb = L.max_batch;
  int* row_req = t + 16;
  int* row_pos = t + 16 + L.m_step;
  int* off = t + 16 + 2 * L.m_step;
  int* nr = off + mb;
  int* len = nr + mb;
  int* bs = len + mb;
  int* act = bs + mb;
  int* blk = act + mb;
  int rows = 0;
  for (int r = 0; r < mb; ++r) {
    off[r] = rows;
    nr[r] = 0;
    len[r] = 0;
    bs[r] = 0;
    act[r] = 0;
    blk[r] = 0;
    if (r >= c->batch) continue;
    blk[r] = c->blk[r];
    len[r] = c->Lr[r];
    bs[r] = c->P[r] + c->blk[r] * L.B;
    if (c->finished[r] || !c->refreshed[r]) continue;
    const int lo = std::max(0, bs[r] - L.w);
    const int hi = std::min(c->Lr[r], bs[r] + L.B + L.w);
    act[r] = 1;
    nr[r] = hi - lo;
    for (int i = 0; i < hi - lo; ++i) {
      row_req[rows + i] = r;
      row_pos[rows + i] = lo + i;
    }
    rows += hi - lo;
  }
  t[0] = rows;
  t[1] = c->batch * L.B;   // LM-head rows
  HIP_TRY(hipMemcpyAsync(c->at<int>(L.off_tab_step), t, (size_t)L.tab_ints_step * 4,
                         hipMemcpyHostToDevice, c->stream));
  HIP_TRY(hipEventRecord(c->ev_step_upload, c->stream));
  c->step_dirty = false;
  return DINFER_OK;
}

// One pass of the model over the rows of a table: embed, every layer with the
// KV scatter before attention, and for a step the final norm, LM head and
// vocab statistics.
dinfer_status run_pass(dinfer_ctx* c, bool step) {
  const Layout& L = c->L;
  const DType dt = L.dt;
  const size_t es = dtype_size(dt);
  hipStream_t st = c->st;
  const int m_cap = step ? L.m_step : c->ref_mcap;
  int* tab = c->at<int>(step ? L.off_tab_step : L.off_tab_ref);
  const PassTable tb = table_view(tab, step ? L.m_step : L.m_ref, L.max_batch);
  GemmPlan gq = step ? L.g_qkv_s : c->ref_q;
  GemmPlan go = step ? L.g_o_s : c->ref_o;
  GemmPlan gg = step ? L.g_gu_s : c->ref_g;
  GemmPlan gd = step ? L.g_d_s : c->ref_d;
  const uint32_t hi_only = step ? c->hi_only_step : c->hi_only_refresh;
  gq.lo = !(hi_only & 1u);
  go.lo = !(hi_only & 2u);
  gg.lo = !(hi_only & 4u);
  gd.lo = !(hi_only & 8u);
  // A dense bf16 model's many-row passes hand the projections their inputs
  // as bf16 hi/lo planes, split once by the kernel that produces them (the
  // norms, the attention, SwiGLU) instead of by every column tile of the fat
  // projection; the planes take the fp32 buffer's bytes.  (An MoE layer's
  // router and expert gathers read the fp32 rows.)
  const bool planes = !L.moe && dt == DType::BF16 && gq.kind == 1;
  gq.ap = go.ap = gg.ap = gd.ap = planes;
  const AttnPlan& ap = step ? L.a_step : L.a_ref;
  const int d = L.d;
  const int F = L.moe ? L.Fs : L.F;   // dense FFN, or the MoE layer's shared expert
  // partial splits the next reader of x still has to add (0 after an MoE combine)
  const int x_splits = L.moe ? 0 : gd.splits;
  float* x = c->at<float>(L.off_x);
  float* a = c->at<float>(L.off_a);
  float* q = c->at<float>(L.off_q);
  float* o = c->at<float>(L.off_o);
  float* act = c->at<float>(L.off_act);
  float* part = c->at<float>(L.off_part);
  const size_t stride_q = (size_t)m_cap * 3 * d, stride_d = (size_t)m_cap * d,
               stride_g = (size_t)m_cap * 2 * F;
  const size_t aps_d = planes ? (size_t)m_cap * d : 0, aps_f = planes ? (size_t)m_cap * F : 0;

  if (step)
    HIP_TRY(launch_step_gate(c->batch, tab, tab + 1, const_cast<int*>(tb.req_nrows), tb.req_active,
                             c->at<int>(L.off_done), st));
  HIP_TRY(launch_embed(dt, tb, m_cap, c->tokens, L.max_len, c->tok_emb, d, L.V, c->m.mask_id,
                       step ? c->dc.smooth_alpha : 0.f, c->at<int>(L.off_sid),
                       c->at<float>(L.off_sp), c->at<uint8_t>(L.off_sv), L.B, x, st));
  for (int l = 0; l < L.nl; ++l) {
    const bool last = l == L.nl - 1;
    HIP_TRY(launch_add_rmsnorm(dt, tb.nrows, m_cap, x, part, l == 0 ? 0 : x_splits, stride_d,
                               c->attn_norm[l], c->m.rms_eps, a, d, st, aps_d));
    HIP_TRY(launch_gemm(gq, dt, a, c->wqkv[l], part, tb.nrows, m_cap, 3 * d, d, st));
    char* kvk = c->at<char>(L.off_kvk) + (size_t)l * L.kv_layer_elems * es;
    char* kvv = c->at<char>(L.off_kvv) + (size_t)l * L.kv_layer_elems * es;
    HIP_TRY(launch_qkv_rope_scatter(dt, tb, m_cap, part, gq.splits, stride_q, d, L.H, L.hd,
                                    c->at<float>(L.off_rope), q, kvk, kvv, L.Lp, st));
    if (!step && last) break;   // a refresh needs only the caches
    HIP_TRY(launch_attention(dt, ap, tb, L.max_batch, m_cap, q, kvk, kvv, L.H, L.hd, L.Lp,
                             c->at<float>(L.off_ao), c->at<float>(L.off_aml), o, st,
                             !(hi_only & 16u), aps_d));
    HIP_TRY(launch_gemm(go, dt, o, c->wo[l], part, tb.nrows, m_cap, d, d, st));
    HIP_TRY(launch_add_rmsnorm(dt, tb.nrows, m_cap, x, part, go.splits, stride_d, c->ffn_norm[l],
                               c->m.rms_eps, a, d, st, aps_d));
    if (!L.moe) {
      if (planes && gg.splits == 1 && gg.nw == 4 && (2 * F) % 256 == 0) {
        // one K split: SwiGLU in the projection's epilogue, act as planes
        HIP_TRY(launch_gemm_fat_swiglu(dt, a, c->wgu[l], act, tb.nrows, m_cap, 2 * F, d, st,
                                       gg.lo != 0));
      } else {
        HIP_TRY(launch_gemm(gg, dt, a, c->wgu[l], part, tb.nrows, m_cap, 2 * F, d, st));
        HIP_TRY(launch_swiglu(tb.nrows, m_cap, part, gg.splits, stride_g, F, act, st, aps_f));
      }
      HIP_TRY(launch_gemm(gd, dt, act, c->wd[l], part, tb.nrows, m_cap, d, F, st));
      continue;
    }
    // MoE layer: route, plan the expert row lists, grouped expert projections,
    // the shared expert, then combine into the residual.
    const int E = L.E, K8 = L.topk, Fe = L.Fe;
    int* sel = c->at<int>(L.off_sel);
    float* gate = c->at<float>(L.off_gate);
    int* pos = c->at<int>(L.off_pos);
    int* row_of = c->at<int>(L.off_rowof);
    int* e_count = c->at<int>(L.off_ecount);
    int* e_off = c->at<int>(L.off_eoff);
    int* n_assign = c->at<int>(L.off_nassign);
    float* egu = c->at<float>(L.off_egu);
    float* eact = c->at<float>(L.off_eact);
    float* ey = c->at<float>(L.off_ey);
    // the shared expert needs only the normalised input: fork it onto the
    // side stream, where it overlaps the router, the plan and the routed
    // experts (it writes part and act, which nothing below touches)
    HIP_TRY(hipEventRecord(c->ev_fork, st));
    HIP_TRY(hipStreamWaitEvent(c->side, c->ev_fork, 0));
    HIP_TRY(launch_gemm(gg, dt, a, c->sgu[l], part, tb.nrows, m_cap, 2 * F, d, c->side));
    HIP_TRY(launch_swiglu(tb.nrows, m_cap, part, gg.splits, stride_g, F, act, c->side));
    HIP_TRY(launch_gemm(gd, dt, act, c->sd[l], part, tb.nrows, m_cap, d, F, c->side));
    HIP_TRY(hipEventRecord(c->ev_join, c->side));
    HIP_TRY(launch_moe_route(dt, tb, m_cap, a, d, c->router[l], E, K8, c->router_bias, L.nl,
                             c->n_bias_blocks, l, sel, gate, c->at<float>(L.off_rlog), st));
    HIP_TRY(launch_moe_plan(tb.nrows, m_cap, sel, E, K8, e_count, e_off, row_of, pos, n_assign, st));
    const void* const* wt = c->at<const void*>(L.off_wtab) + (size_t)l * 2 * E;
    if (c->offload)
      HIP_TRY(launch_expert_usage(e_count, E, c->at<int>(L.off_resident) + (size_t)l * E,
                                  c->at<int>(L.off_eusage) + (size_t)l * E,
                                  c->at<long long>(L.off_eacct) + (size_t)l * 4, st));
    HIP_TRY(launch_gemm_grouped(dt, a, row_of, e_count, e_off, E, m_cap, wt, egu, 2 * Fe, d, st));
    HIP_TRY(launch_swiglu(n_assign, m_cap * K8, egu, 1, 0, Fe, eact, st));
    HIP_TRY(launch_gemm_grouped(dt, eact, nullptr, e_count, e_off, E, m_cap, wt + E, ey, d, Fe,
                                st));
    HIP_TRY(hipStreamWaitEvent(st, c->ev_join, 0));   // join the shared expert
    HIP_TRY(launch_moe_combine(tb.nrows, m_cap, x, part, gd.splits, stride_d, ey, pos, gate, K8, d,
                               st));
  }
  if (!step) return DINFER_OK;
  float* hf = c->at<float>(L.off_hf);
  HIP_TRY(launch_final_norm(dt, tb, L.max_batch, L.B, x, part, x_splits, stride_d, c->final_norm,
                            c->m.rms_eps, hf, d, c->plant_id, c->plant_bias, L.max_len,
                            c->at<int>(L.off_rpid), c->at<float>(L.off_rpb), st));
  // LM head with the vocab statistics in its epilogue: per-(row, column
  // tile) records, then one merge per row; the fp32 logits are stored only
  // while keep_logits is on (inspection)
  VocabEpi ve{};
  ve.row_plant_id = c->at<int>(L.off_rpid);
  ve.row_plant_bias = c->at<float>(L.off_rpb);
  ve.mask_id = c->m.mask_id;
  ve.logits = c->keep_logits ? c->at<float>(L.off_logits) : nullptr;
  ve.rec_f = c->at<float>(L.off_lmrec);
  ve.rec_i = reinterpret_cast<int*>(ve.rec_f + (size_t)L.lm_rows * L.lm_tiles * (2 + 8));
  ve.n_tiles = L.lm_tiles;
  HIP_TRY(launch_gemm_lmhead(L.g_lm, dt, hf, c->lm_head, tab + 1, L.lm_rows, L.V, d, ve, st));
  HIP_TRY(launch_vocab_merge_tiles(c->batch * L.B, L.lm_tiles, ve.rec_f, ve.rec_i,
                                   c->at<int>(L.off_argmax), c->at<float>(L.off_conf),
                                   c->at<float>(L.off_lse), c->at<int>(L.off_tid),
                                   c->at<float>(L.off_tp), st));
  return DINFER_OK;
}

dinfer_status launch_commit_step(dinfer_ctx* c) {
  const Layout& L = c->L;
  const PassTable tb = table_view(c->at<int>(L.off_tab_step), L.m_step, L.max_batch);
  CommitArgs a{};
  a.batch = c->batch;
  a.B = L.B;
  a.max_len = L.max_len;
  a.mask_id = c->m.mask_id;
  a.hierarchical = c->dc.hierarchical;
  a.tau = c->dc.tau;
  a.kappa = c->dc.credit_kappa;
  a.gamma = c->dc.credit_decay;
  a.lambda = c->dc.credit_weight;
  a.req_bs = tb.req_bs;
  a.req_active = tb.req_active;
  a.req_len = tb.req_len;
  a.req_blk = tb.req_blk;
  a.eos_id = c->dc.eos_id;
  a.tokens = c->tokens;
  a.argmax = c->at<int>(L.off_argmax);
  a.conf = c->at<float>(L.off_conf);
  a.topk_id = c->at<int>(L.off_tid);
  a.topk_p = c->at<float>(L.off_tp);
  a.credit = c->at<float>(L.off_credit);
  a.tracked = c->at<int>(L.off_tracked);
  a.smooth_id = c->at<int>(L.off_sid);
  a.smooth_p = c->at<float>(L.off_sp);
  a.smooth_valid = c->at<uint8_t>(L.off_sv);
  a.commit_mask = c->at<uint8_t>(L.off_cm);
  a.block_done = c->at<int>(L.off_done);
  a.step_count = c->at<int>(L.off_steps);
  a.commit_count = c->at<int>(L.off_ccount);
  a.decode_stats = c->at<int>(L.off_dstat);
  HIP_TRY(launch_commit(a, c->st));
  return DINFER_OK;
}

int unfinished(const dinfer_ctx* c) {
  int n = 0;
  for (int r = 0; r < c->batch; ++r) n += !c->finished[r];
  return n;
}

int active_count(const dinfer_ctx* c) {
  int n = 0;
  for (int r = 0; r < c->batch; ++r) n += (!c->finished[r] && c->refreshed[r]);
  return n;
}

size_t expert_gu_bytes(const Layout& L) { return (size_t)2 * L.Fe * L.d * dtype_size(L.dt); }
size_t expert_dn_bytes(const Layout& L) { return (size_t)L.d * L.Fe * dtype_size(L.dt); }

// Expert e of layer l into HBM slot s (host store -> slot copy on the
// context's stream, after every kernel enqueued before it), and the host
// staging of its table entries and residency.
dinfer_status move_expert_in(dinfer_ctx* c, int l, int e, int s) {
  const Layout& L = c->L;
  const size_t gu = expert_gu_bytes(L), dn = expert_dn_bytes(L);
  char* dst = c->d_slots + ((size_t)l * c->slots + s) * (gu + dn);
  HIP_TRY(hipMemcpyAsync(dst, c->h_gu[l] + e * gu, gu, hipMemcpyHostToDevice, c->stream));
  HIP_TRY(hipMemcpyAsync(dst + gu, c->h_dn[l] + e * dn, dn, hipMemcpyHostToDevice, c->stream));
  c->h_wtab[((size_t)l * 2 + 0) * L.E + e] = dst;
  c->h_wtab[((size_t)l * 2 + 1) * L.E + e] = dst + gu;
  c->h_resident[(size_t)l * L.E + e] = 1;
  c->slot_expert[l][s] = e;
  c->bytes_h2d += (long long)(gu + dn);
  return DINFER_OK;
}

// Expert e of layer l back to its host-store address (read by the kernels
// from pinned host memory).
void move_expert_out(dinfer_ctx* c, int l, int e) {
  const Layout& L = c->L;
  const size_t gu = expert_gu_bytes(L), dn = expert_dn_bytes(L);
  c->h_wtab[((size_t)l * 2 + 0) * L.E + e] = c->hd_gu[l] + e * gu;
  c->h_wtab[((size_t)l * 2 + 1) * L.E + e] = c->hd_dn[l] + e * dn;
  c->h_resident[(size_t)l * L.E + e] = 0;
}

dinfer_status upload_expert_tables(dinfer_ctx* c, bool reset_usage) {
  const Layout& L = c->L;
  const size_t ne = (size_t)L.nl * L.E;
  HIP_TRY(hipMemcpyAsync(c->at<char>(L.off_wtab), c->h_wtab, ne * 2 * sizeof(void*),
                         hipMemcpyHostToDevice, c->stream));
  HIP_TRY(hipMemcpyAsync(c->at<char>(L.off_resident), c->h_resident, ne * 4,
                         hipMemcpyHostToDevice, c->stream));
  if (reset_usage) HIP_TRY(hipMemsetAsync(c->at<char>(L.off_eusage), 0, ne * 4, c->stream));
  return DINFER_OK;
}

// Interval placement (TIDE abstract: expert activations are stable within a
// block, so the placement is refreshed per interval): per layer, the `slots`
// experts with the most row assignments become resident (ties: the resident
// one, then the lower id); only the experts that change are copied, each into
// the slot of an expert that leaves.  The counts run from one block-start
// placement to the next (block_start: the refresh just run and the steps
// since the last block start; then they restart), so a placement inside a
// block ranks by everything the block has routed so far, not by its last
// few steps (ranked by the interval alone, the mid-block placements evicted
// experts the block still needed: 48 slots, every 4 steps, 1.9 GB read from
// host against 0.2 GB with block-start placement only).
dinfer_status place_experts(dinfer_ctx* c, bool block_start) {
  const Layout& L = c->L;
  const int E = L.E, C = c->slots;
  std::vector<int> cnt((size_t)L.nl * E);
  HIP_TRY(hipMemcpyAsync(cnt.data(), c->at<int>(L.off_eusage), cnt.size() * 4,
                         hipMemcpyDeviceToHost, c->stream));
  HIP_TRY(hipStreamSynchronize(c->stream));   // also: the last table upload has been read
  for (int l = 0; l < L.nl; ++l) {
    const int* u = cnt.data() + (size_t)l * E;
    const int* res = c->h_resident + (size_t)l * E;
    std::vector<int> order(E);
    for (int e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
      if (u[a] != u[b]) return u[a] > u[b];
      return res[a] > res[b];
    });
    std::vector<uint8_t> want(E, 0);
    for (int i = 0; i < C; ++i) want[order[i]] = 1;
    std::vector<int> in;
    for (int e = 0; e < E; ++e)
      if (want[e] && !res[e]) in.push_back(e);
    size_t k = 0;
    for (int s = 0; s < C && k < in.size(); ++s) {
      const int out = c->slot_expert[l][s];
      if (want[out]) continue;
      move_expert_out(c, l, out);
      dinfer_status st = move_expert_in(c, l, in[k++], s);
      if (st != DINFER_OK) return st;
    }
  }
  c->placements += 1;
  c->steps_since_place = 0;
  return upload_expert_tables(c, block_start);
}

}  // namespace

// ----------------------------------------------------------------------------
extern "C" {

const char* dinfer_status_str(dinfer_status s) {
  switch (s) {
    case DINFER_OK: return "DINFER_OK";
    case DINFER_E_ARG: return "DINFER_E_ARG";
    case DINFER_E_WORKSPACE: return "DINFER_E_WORKSPACE";
    case DINFER_E_STATE: return "DINFER_E_STATE";
    case DINFER_E_HIP: return "DINFER_E_HIP";
    case DINFER_E_UNSUPPORTED: return "DINFER_E_UNSUPPORTED";
  }
  return "DINFER_E_UNKNOWN";
}

const char* dinfer_last_error(void) { return g_last_error.c_str(); }

size_t dinfer_workspace_bytes(const dinfer_model_cfg* m, const dinfer_decode_cfg* dc,
                              int32_t max_batch, int32_t max_len) {
  Layout L;
  if (!make_layout(m, dc, max_batch, max_len, &L, nullptr)) return 0;
  return L.total;
}

dinfer_status dinfer_step_init(const dinfer_model_cfg* m, const dinfer_decode_cfg* dc,
                               const dinfer_weights* w, int32_t max_batch, int32_t max_len,
                               void* d_workspace, size_t ws_bytes, void* stream,
                               dinfer_ctx** out) {
  if (!out) return fail(DINFER_E_ARG, "out is null");
  *out = nullptr;
  std::string why;
  Layout L;
  if (!make_layout(m, dc, max_batch, max_len, &L, &why)) {
    const bool unsup = why.find("not supported") != std::string::npos ||
                       why.find("must be 64 or 128") != std::string::npos ||
                       why.find("GEMM shapes") != std::string::npos;
    return fail(unsup ? DINFER_E_UNSUPPORTED : DINFER_E_ARG, why);
  }
  if (!w || !w->tok_emb || !w->final_norm || !w->lm_head || !w->attn_norm || !w->wqkv || !w->wo ||
      !w->ffn_norm)
    return fail(DINFER_E_ARG, "missing weight pointers");
  // MoE experts may be left out (both arrays NULL) when an expert cache will
  // hold them (dinfer_expert_offload)
  const bool have_experts = L.moe && w->exp_gate_up && w->exp_down;
  if (L.moe ? (!w->router || !w->shared_gate_up || !w->shared_down ||
               (!w->exp_gate_up != !w->exp_down))
            : (!w->w_gate_up || !w->w_down))
    return fail(DINFER_E_ARG, "missing FFN weight pointers");
  for (int l = 0; l < m->n_layers; ++l) {
    bool ok = w->attn_norm[l] && w->wqkv[l] && w->wo[l] && w->ffn_norm[l];
    if (L.moe)
      ok = ok && w->router[l] && w->shared_gate_up[l] && w->shared_down[l] &&
           (!have_experts || (w->exp_gate_up[l] && w->exp_down[l]));
    else
      ok = ok && w->w_gate_up[l] && w->w_down[l];
    if (!ok) return fail(DINFER_E_ARG, "missing per-layer weight pointer at layer " + std::to_string(l));
  }
  if (!d_workspace) return fail(DINFER_E_WORKSPACE, "workspace is null");
  if (reinterpret_cast<uintptr_t>(d_workspace) % kAlign != 0)
    return fail(DINFER_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(DINFER_E_WORKSPACE, "workspace too small: need " + std::to_string(L.total) +
                                        " bytes, got " + std::to_string(ws_bytes));

  dinfer_ctx* c = new dinfer_ctx();
  c->m = *m;
  c->dc = *dc;
  c->L = L;
  c->stream = static_cast<hipStream_t>(stream);
  c->st = c->stream;
  c->ws = static_cast<char*>(d_workspace);
  c->tok_emb = w->tok_emb;
  c->final_norm = w->final_norm;
  c->lm_head = w->lm_head;
  c->attn_norm.assign(w->attn_norm, w->attn_norm + m->n_layers);
  c->wqkv.assign(w->wqkv, w->wqkv + m->n_layers);
  c->wo.assign(w->wo, w->wo + m->n_layers);
  c->ffn_norm.assign(w->ffn_norm, w->ffn_norm + m->n_layers);
  if (L.moe) {
    c->router.assign(w->router, w->router + m->n_layers);
    if (have_experts) {
      c->egu.assign(w->exp_gate_up, w->exp_gate_up + m->n_layers);
      c->ed.assign(w->exp_down, w->exp_down + m->n_layers);
    }
    c->sgu.assign(w->shared_gate_up, w->shared_gate_up + m->n_layers);
    c->sd.assign(w->shared_down, w->shared_down + m->n_layers);
  } else {
    c->wgu.assign(w->w_gate_up, w->w_gate_up + m->n_layers);
    c->wd.assign(w->w_down, w->w_down + m->n_layers);
  }

  auto cleanup = [&](dinfer_status s) {
    dinfer_destroy(c);
    return s;
  };
  if (hipHostMalloc(&c->h_tab_step, (size_t)L.tab_ints_step * 4) != hipSuccess ||
      hipHostMalloc(&c->h_tab_ref, (size_t)L.tab_ints_ref * 4) != hipSuccess ||
      hipHostMalloc(&c->h_misc, 64 * 4) != hipSuccess)
    return cleanup(fail(DINFER_E_HIP, "pinned host staging allocation failed"));
  if (hipEventCreateWithFlags(&c->ev_step_upload, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->ev_ref_upload, hipEventDisableTiming) != hipSuccess ||
      hipEventCreate(&c->ev0) != hipSuccess || hipEventCreate(&c->ev1) != hipSuccess)
    return cleanup(fail(DINFER_E_HIP, "event creation failed"));
  std::memset(c->h_tab_step, 0, (size_t)L.tab_ints_step * 4);
  std::memset(c->h_tab_ref, 0, (size_t)L.tab_ints_ref * 4);
  if (L.moe) {
    if (hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming) != hipSuccess)
      return cleanup(fail(DINFER_E_HIP, "stream or event creation failed"));
    const size_t ne = (size_t)L.nl * L.E;
    if (hipHostMalloc(&c->h_wtab, ne * 2 * sizeof(void*)) != hipSuccess ||
        hipHostMalloc(&c->h_resident, ne * 4) != hipSuccess)
      return cleanup(fail(DINFER_E_HIP, "pinned host staging allocation failed"));
    std::memset(c->h_wtab, 0, ne * 2 * sizeof(void*));
    for (size_t i = 0; i < ne; ++i) c->h_resident[i] = 1;
    if (have_experts) {
      // every expert in HBM: expert e of a layer at base + e * (its matrix bytes)
      const size_t es = dtype_size(L.dt);
      const size_t gu = (size_t)2 * L.Fe * L.d * es, dn = (size_t)L.d * L.Fe * es;
      for (int l = 0; l < L.nl; ++l)
        for (int e = 0; e < L.E; ++e) {
          c->h_wtab[((size_t)l * 2 + 0) * L.E + e] = static_cast<const char*>(c->egu[l]) + e * gu;
          c->h_wtab[((size_t)l * 2 + 1) * L.E + e] = static_cast<const char*>(c->ed[l]) + e * dn;
        }
      c->experts_ready = true;
    }
    if (hipMemcpyAsync(c->at<char>(L.off_wtab), c->h_wtab, ne * 2 * sizeof(void*),
                       hipMemcpyHostToDevice, c->stream) != hipSuccess ||
        hipMemcpyAsync(c->at<char>(L.off_resident), c->h_resident, ne * 4, hipMemcpyHostToDevice,
                       c->stream) != hipSuccess ||
        hipMemsetAsync(c->at<char>(L.off_eusage), 0, ne * 4, c->stream) != hipSuccess ||
        hipMemsetAsync(c->at<char>(L.off_eacct), 0, (size_t)L.nl * 4 * 8, c->stream) != hipSuccess)
      return cleanup(fail(DINFER_E_HIP, "expert table upload failed"));
  } else {
    c->experts_ready = true;
  }

  // RoPE table [pos][cos(0..hd/2) | sin(0..hd/2)], angles in fp64.
  std::vector<float> cs((size_t)max_len * L.hd);
  const int half = L.hd / 2;
  for (int p = 0; p < max_len; ++p)
    for (int j = 0; j < half; ++j) {
      const double ang = (double)p * std::pow((double)m->rope_theta, -2.0 * j / L.hd);
      cs[(size_t)p * L.hd + j] = (float)std::cos(ang);
      cs[(size_t)p * L.hd + half + j] = (float)std::sin(ang);
    }
  if (hipMemcpyAsync(c->at<float>(L.off_rope), cs.data(), cs.size() * 4, hipMemcpyHostToDevice,
                     c->stream) != hipSuccess ||
      hipMemsetAsync(c->at<char>(L.off_done), 0, (size_t)max_batch * 4, c->stream) != hipSuccess ||
      hipMemsetAsync(c->at<char>(L.off_steps), 0, (size_t)max_batch * 4, c->stream) != hipSuccess ||
      hipMemsetAsync(c->at<char>(L.off_ccount), 0, (size_t)max_batch * 4, c->stream) != hipSuccess ||
      hipMemsetAsync(c->at<char>(L.off_dstat), 0, (size_t)max_batch * kDecodeStatWords * 4,
                     c->stream) != hipSuccess ||
      hipMemsetAsync(c->at<char>(L.off_tab_step), 0, (size_t)L.tab_ints_step * 4, c->stream) !=
          hipSuccess ||
      hipMemsetAsync(c->at<char>(L.off_tab_ref), 0, (size_t)L.tab_ints_ref * 4, c->stream) !=
          hipSuccess ||
      // cache padding and positions never written must hold finite values:
      // the attention multiplies their (zero) probabilities with V
      hipMemsetAsync(c->at<char>(L.off_kvk), 0, L.kv_layer_elems * L.nl * dtype_size(L.dt),
                     c->stream) != hipSuccess ||
      hipMemsetAsync(c->at<char>(L.off_kvv), 0, L.kv_layer_elems * L.nl * dtype_size(L.dt),
                     c->stream) != hipSuccess ||
      hipStreamSynchronize(c->stream) != hipSuccess)
    return cleanup(fail(DINFER_E_HIP, "workspace initialisation failed"));
  *out = c;
  return DINFER_OK;
}

dinfer_status dinfer_set_batch(dinfer_ctx* c, int32_t batch, int32_t* d_tokens,
                               const int32_t* h_prompt_len, const int32_t* h_gen_len,
                               const int32_t* d_plant_id, const float* d_plant_bias,
                               const float* d_router_bias) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  if (batch < 1 || batch > c->L.max_batch) return fail(DINFER_E_ARG, "batch out of range");
  if (!d_tokens || !h_prompt_len || !h_gen_len) return fail(DINFER_E_ARG, "null batch pointer");
  if (d_router_bias && !c->L.moe) return fail(DINFER_E_ARG, "router bias given for a dense model");
  const int B = c->L.B;
  for (int r = 0; r < batch; ++r) {
    if (h_prompt_len[r] < 0 || h_gen_len[r] < B || h_gen_len[r] % B != 0)
      return fail(DINFER_E_ARG, "gen_len must be a positive multiple of block_len");
    if (h_prompt_len[r] + h_gen_len[r] > c->L.max_len)
      return fail(DINFER_E_ARG, "prompt_len + gen_len exceeds max_len");
  }
  if (c->graph && (batch != c->batch || d_tokens != c->tokens || d_plant_id != c->plant_id ||
                   d_plant_bias != c->plant_bias)) {
    // kernel arguments captured in the graph change with these
    (void)hipGraphExecDestroy(c->graph);
    c->graph = nullptr;
    c->graph_steps = 0;
  }
  int nb = 0;
  for (int r = 0; r < batch; ++r) nb = std::max(nb, h_gen_len[r] / B);
  if (c->graph && (d_router_bias != c->router_bias || nb != c->n_bias_blocks)) {
    (void)hipGraphExecDestroy(c->graph);
    c->graph = nullptr;
    c->graph_steps = 0;
  }
  c->batch = batch;
  c->tokens = d_tokens;
  c->plant_id = d_plant_id;
  c->plant_bias = d_plant_bias;
  c->router_bias = d_router_bias;
  c->n_bias_blocks = nb;
  c->P.assign(h_prompt_len, h_prompt_len + batch);
  c->G.assign(h_gen_len, h_gen_len + batch);
  c->Lr.resize(batch);
  c->blk.assign(batch, 0);
  c->nblk.resize(batch);
  for (int r = 0; r < batch; ++r) {
    c->Lr[r] = c->P[r] + c->G[r];
    c->nblk[r] = c->G[r] / B;
  }
  c->finished.assign(batch, 0);
  c->refreshed.assign(batch, 0);
  c->step_dirty = true;
  c->stats_ready = false;
  c->state = 1;
  const Layout& L = c->L;
  HIP_TRY(hipMemsetAsync(c->at<char>(L.off_done), 0, (size_t)L.max_batch * 4, c->stream));
  HIP_TRY(hipMemsetAsync(c->at<char>(L.off_steps), 0, (size_t)L.max_batch * 4, c->stream));
  HIP_TRY(hipMemsetAsync(c->at<char>(L.off_ccount), 0, (size_t)L.max_batch * 4, c->stream));
  HIP_TRY(hipMemsetAsync(c->at<char>(L.off_dstat), 0, (size_t)L.max_batch * kDecodeStatWords * 4,
                         c->stream));
  return upload_step_table(c);
}

dinfer_status dinfer_refill(dinfer_ctx* c, int32_t slot, int32_t prompt_len, int32_t gen_len) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  if (c->state < 1) return fail(DINFER_E_STATE, "refill before set_batch");
  if (slot < 0 || slot >= c->batch) return fail(DINFER_E_ARG, "slot out of range");
  if (!c->finished[slot]) return fail(DINFER_E_STATE, "slot has not finished");
  const int B = c->L.B;
  if (prompt_len < 0 || gen_len < B || gen_len % B != 0)
    return fail(DINFER_E_ARG, "gen_len must be a positive multiple of block_len");
  if (prompt_len + gen_len > c->L.max_len)
    return fail(DINFER_E_ARG, "prompt_len + gen_len exceeds max_len");
  if (c->router_bias && gen_len / B > c->n_bias_blocks)
    return fail(DINFER_E_ARG, "more blocks than the router bias holds");
  c->P[slot] = prompt_len;
  c->G[slot] = gen_len;
  c->Lr[slot] = prompt_len + gen_len;
  c->nblk[slot] = gen_len / B;
  c->blk[slot] = 0;
  c->finished[slot] = 0;
  c->refreshed[slot] = 0;
  c->step_dirty = true;
  c->stats_ready = false;
  const Layout& L = c->L;
  HIP_TRY(hipMemsetAsync(c->at<int>(L.off_done) + slot, 0, 4, c->stream));
  HIP_TRY(hipMemsetAsync(c->at<int>(L.off_steps) + slot, 0, 4, c->stream));
  HIP_TRY(hipMemsetAsync(c->at<int>(L.off_ccount) + slot, 0, 4, c->stream));
  HIP_TRY(hipMemsetAsync(c->at<int>(L.off_dstat) + (size_t)slot * kDecodeStatWords, 0,
                         kDecodeStatWords * 4, c->stream));
  return DINFER_OK;
}

dinfer_status dinfer_finished(const dinfer_ctx* c, uint8_t* h_finished) {
  if (!c || !h_finished) return fail(DINFER_E_ARG, "null argument");
  for (int r = 0; r < c->batch; ++r) h_finished[r] = c->finished[r] ? 1 : 0;
  return DINFER_OK;
}

dinfer_status dinfer_pending_rows(const dinfer_ctx* c, int32_t* h_decode_rows,
                                  int32_t* h_refresh_rows) {
  if (!c || !h_decode_rows || !h_refresh_rows) return fail(DINFER_E_ARG, "null argument");
  if (c->state < 1) return fail(DINFER_E_STATE, "pending_rows before set_batch");
  const Layout& L = c->L;
  for (int r = 0; r < c->batch; ++r) {
    h_decode_rows[r] = h_refresh_rows[r] = 0;
    if (c->finished[r]) continue;
    if (!c->refreshed[r]) {
      h_refresh_rows[r] = c->Lr[r];
      continue;
    }
    const int bs = c->P[r] + c->blk[r] * L.B;
    h_decode_rows[r] = std::min(c->Lr[r], bs + L.B + L.w) - std::max(0, bs - L.w);
  }
  return DINFER_OK;
}

// Deficit token-budget admission (host only).  The queue holds the waiting
// slots first come first served; `queued` mirrors membership.
struct dinfer_sched {
  int64_t budget = 0;
  int n = 0;
  int64_t deficit = 0;
  std::deque<int> queue;
  std::vector<uint8_t> queued;
};

dinfer_status dinfer_sched_create(int64_t token_budget, int32_t n_slots, dinfer_sched** out) {
  if (!out) return fail(DINFER_E_ARG, "out is null");
  *out = nullptr;
  if (token_budget < 0 || token_budget > kSchedMaxBudget)
    return fail(DINFER_E_ARG, "token_budget out of [0, 2^62]");
  if (n_slots < 1) return fail(DINFER_E_ARG, "n_slots < 1");
  dinfer_sched* s = new (std::nothrow) dinfer_sched;
  if (!s) return fail(DINFER_E_ARG, "out of host memory");
  s->budget = token_budget;
  s->n = n_slots;
  s->queued.assign(n_slots, 0);
  *out = s;
  return DINFER_OK;
}

void dinfer_sched_destroy(dinfer_sched* s) { delete s; }

dinfer_status dinfer_sched_round(dinfer_sched* s, const int32_t* h_decode_rows,
                                 const int32_t* h_refresh_rows, uint8_t* h_admit,
                                 int64_t* h_deficit) {
  if (!s || !h_decode_rows || !h_refresh_rows || !h_admit) return fail(DINFER_E_ARG, "null argument");
  int64_t dec = 0;
  for (int r = 0; r < s->n; ++r) {
    if (h_decode_rows[r] < 0 || h_refresh_rows[r] < 0)
      return fail(DINFER_E_ARG, "negative row count");
    if (h_decode_rows[r] > 0 && h_refresh_rows[r] > 0)
      return fail(DINFER_E_ARG, "a slot both decodes and waits for a refresh");
    dec += h_decode_rows[r];
  }
  // slots that stopped waiting leave; this round's arrivals join in slot order
  std::deque<int> q;
  for (int r : s->queue) {
    if (h_refresh_rows[r] > 0) q.push_back(r);
    else s->queued[r] = 0;
  }
  for (int r = 0; r < s->n; ++r)
    if (h_refresh_rows[r] > 0 && !s->queued[r]) {
      q.push_back(r);
      s->queued[r] = 1;
    }
  // the decodes spend the round's budget first; whole refreshes follow while
  // the counter covers them (the head once in a round with no decode)
  s->deficit += s->budget - dec;
  std::memset(h_admit, 0, (size_t)s->n);
  bool admitted = false;
  while (!q.empty()) {
    const int head = q.front();
    const int64_t cost = h_refresh_rows[head];
    if (s->deficit < cost && (dec > 0 || admitted)) break;
    h_admit[head] = 1;
    s->deficit -= cost;
    s->queued[head] = 0;
    q.pop_front();
    admitted = true;
  }
  if (q.empty()) s->deficit = 0;   // the counter runs only while a refresh waits
  s->queue.swap(q);
  if (h_deficit) *h_deficit = s->deficit;
  return DINFER_OK;
}

dinfer_status dinfer_refresh_kv(dinfer_ctx* c, const uint8_t* h_req_mask) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  if (c->state < 1) return fail(DINFER_E_STATE, "refresh_kv before set_batch");
  if (!c->experts_ready)
    return fail(DINFER_E_STATE, "no expert weights: give them at init or call dinfer_expert_offload");
  const Layout& L = c->L;
  HIP_TRY(hipEventSynchronize(c->ev_ref_upload));
  int* t = c->h_tab_ref;
  const int mb = L.max_batch;
  int* row_req = t + 16;
  int* row_pos = t + 16 + L.m_ref;
  int* off = t + 16 + 2 * L.m_ref;
  int* nr = off + mb;
  int* len = nr + mb;
  int* bs = len + mb;
  int* act = bs + mb;
  int* blk = act + mb;
  int* mask = c->h_misc;
  int rows = 0, nsel = 0;
  for (int r = 0; r < mb; ++r) {
    off[r] = rows;
    nr[r] = len[r] = bs[r] = act[r] = blk[r] = 0;
    mask[r] = 0;
    if (r >= c->batch || c->finished[r]) continue;
    if (h_req_mask && !h_req_mask[r]) continue;
    mask[r] = 1;
    ++nsel;
    blk[r] = c->blk[r];
    len[r] = c->Lr[r];
    bs[r] = c->P[r] + c->blk[r] * L.B;
    act[r] = 1;
    nr[r] = c->Lr[r];
    for (int i = 0; i < c->Lr[r]; ++i) {
      row_req[rows + i] = r;
      row_pos[rows + i] = i;
    }
    rows += c->Lr[r];
  }
  if (nsel == 0) return DINFER_OK;
  t[0] = rows;
  // plans for this call's rows (K splits that suit the actual tile count),
  // unless their partials would not fit the buffer sized for m_ref
  {
    const int d = L.d, Fd = L.moe ? L.Fs : L.F;
    int m_eff = std::min(L.m_ref, (rows + 15) / 16 * 16);
    GemmPlan pq = plan_gemm(L.dt, m_eff, 3 * d, d, 256), po = plan_gemm(L.dt, m_eff, d, d, 256),
             pg = plan_gemm(L.dt, m_eff, 2 * Fd, d, 256), pd = plan_gemm(L.dt, m_eff, d, Fd, 256);
    auto fits = [&](const GemmPlan& g, int N) {
      return (size_t)g.splits * m_eff * N <= L.part_elems;
    };
    if (!(fits(pq, 3 * d) && fits(po, d) && fits(pg, 2 * Fd) && fits(pd, d))) {
      m_eff = L.m_ref;
      pq = L.g_qkv_r, po = L.g_o_r, pg = L.g_gu_r, pd = L.g_d_r;
    }
    for (GemmPlan* g : {&pq, &po, &pg, &pd})   // buffers hold m_all rows
      g->guard = g->kind == 0 && g->mtiles > 1 && L.m_all < 16 * g->mt * g->mtiles;
    c->ref_mcap = m_eff;
    c->ref_q = pq, c->ref_o = po, c->ref_g = pg, c->ref_d = pd;
  }
  HIP_TRY(hipMemcpyAsync(c->at<int>(L.off_tab_ref), t, (size_t)L.tab_ints_ref * 4,
                         hipMemcpyHostToDevice, c->stream));
  HIP_TRY(hipMemcpyAsync(c->at<int>(L.off_mask), mask, (size_t)mb * 4, hipMemcpyHostToDevice,
                         c->stream));
  HIP_TRY(hipEventRecord(c->ev_ref_upload, c->stream));
  c->st = c->stream;
  dinfer_status s = run_pass(c, false);
  if (s != DINFER_OK) return s;
  HIP_TRY(launch_block_reset(mb, L.B, c->at<int>(L.off_mask), c->at<float>(L.off_credit),
                             c->at<int>(L.off_tracked), c->at<uint8_t>(L.off_sv),
                             c->at<uint8_t>(L.off_cm), c->at<int>(L.off_done),
                             c->at<int>(L.off_steps), c->stream));
  for (int r = 0; r < c->batch; ++r)
    if (mask[r]) c->refreshed[r] = 1;
  c->step_dirty = true;
  c->stats_ready = false;   // a refreshed block starts over: the last stats are stale
  return DINFER_OK;
}

dinfer_status dinfer_denoise_step(dinfer_ctx* c) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  if (c->state < 1) return fail(DINFER_E_STATE, "denoise_step before set_batch");
  if (active_count(c) == 0) return fail(DINFER_E_STATE, "no refreshed request with an open block");
  if (c->step_dirty) {
    dinfer_status s = upload_step_table(c);
    if (s != DINFER_OK) return s;
  }
  c->st = c->stream;
  dinfer_status s = run_pass(c, true);
  if (s == DINFER_OK) c->stats_ready = true;
  return s;
}

dinfer_status dinfer_commit(dinfer_ctx* c) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  if (!c->stats_ready) return fail(DINFER_E_STATE, "commit without a preceding denoise_step");
  c->st = c->stream;
  dinfer_status s = launch_commit_step(c);
  if (s == DINFER_OK) c->stats_ready = false;
  return s;
}

dinfer_status dinfer_advance_blocks(dinfer_ctx* c, uint8_t* h_needs_refresh, int32_t* h_unfinished) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  if (c->state < 1) return fail(DINFER_E_STATE, "advance_blocks before set_batch");
  std::vector<int> done(c->batch);
  HIP_TRY(hipMemcpyAsync(done.data(), c->at<int>(c->L.off_done), (size_t)c->batch * 4,
                         hipMemcpyDeviceToHost, c->stream));
  HIP_TRY(hipStreamSynchronize(c->stream));
  c->stats_ready = false;   // blocks may move: a commit needs a fresh denoise_step
  for (int r = 0; r < c->batch; ++r) {
    if (h_needs_refresh) h_needs_refresh[r] = 0;
    if (c->finished[r] || !c->refreshed[r] || !done[r]) continue;
    if (done[r] == 2) {   // end-of-sequence: no masked response position is left
      c->finished[r] = 1;
      c->refreshed[r] = 0;
      c->step_dirty = true;
      continue;
    }
    c->blk[r] += 1;
    c->refreshed[r] = 0;
    c->step_dirty = true;
    if (c->blk[r] >= c->nblk[r]) {
      c->finished[r] = 1;
      c->blk[r] = c->nblk[r] - 1;
    }
  }
  // every unfinished request without a refresh of its current block (one
  // that moved to a new block, or a refilled slot) needs one
  if (h_needs_refresh)
    for (int r = 0; r < c->batch; ++r) h_needs_refresh[r] = !c->finished[r] && !c->refreshed[r];
  if (h_unfinished) *h_unfinished = unfinished(c);
  return DINFER_OK;
}

static dinfer_status capture_graph(dinfer_ctx* c, int U) {
  if (c->graph) {
    (void)hipGraphExecDestroy(c->graph);
    c->graph = nullptr;
  }
  if (!c->cap_stream) HIP_TRY(hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));
  HIP_TRY(hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal));
  c->st = c->cap_stream;
  dinfer_status s = DINFER_OK;
  for (int u = 0; u < U && s == DINFER_OK; ++u) {
    s = run_pass(c, true);
    if (s == DINFER_OK) s = launch_commit_step(c);
  }
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(c->cap_stream, &g);
  c->st = c->stream;
  if (s != DINFER_OK) {
    if (g) (void)hipGraphDestroy(g);
    return s;
  }
  if (e != hipSuccess) return fail(DINFER_E_HIP, std::string("graph capture: ") + hipGetErrorString(e));
  e = hipGraphInstantiate(&c->graph, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) return fail(DINFER_E_HIP, std::string("graph instantiate: ") + hipGetErrorString(e));
  c->graph_steps = U;
  return DINFER_OK;
}

dinfer_status dinfer_step_graph(dinfer_ctx* c, int32_t n_steps) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  const int U = c->dc.graph_unroll;
  if (U <= 0) return fail(DINFER_E_STATE, "graph_unroll is 0: no step graph");
  if (n_steps < 0 || n_steps % U != 0)
    return fail(DINFER_E_ARG, "n_steps must be a non-negative multiple of graph_unroll");
  if (c->state < 1) return fail(DINFER_E_STATE, "step_graph before set_batch");
  if (active_count(c) == 0) return fail(DINFER_E_STATE, "no refreshed request with an open block");
  if (c->step_dirty) {
    dinfer_status s = upload_step_table(c);
    if (s != DINFER_OK) return s;
  }
  if (!c->graph || c->graph_steps != U) {
    dinfer_status s = capture_graph(c, U);
    if (s != DINFER_OK) return s;
  }
  for (int i = 0; i < n_steps / U; ++i) HIP_TRY(hipGraphLaunch(c->graph, c->stream));
  c->stats_ready = false;
  return DINFER_OK;
}

dinfer_status dinfer_run_to_completion(dinfer_ctx* c, int32_t max_steps, dinfer_run_stats* h_stats) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  if (c->state < 1) return fail(DINFER_E_STATE, "run_to_completion before set_batch");
  const auto t0 = std::chrono::steady_clock::now();
  dinfer_run_stats stats{};
  double refresh_ms = 0.0;
  std::vector<uint8_t> need(c->batch);
  auto refresh = [&](const uint8_t* mask) -> dinfer_status {
    int n = 0;
    for (int r = 0; r < c->batch; ++r) n += (!c->finished[r] && !c->refreshed[r] && (!mask || mask[r]));
    if (n == 0) return DINFER_OK;
    std::vector<uint8_t> sel(c->batch);
    for (int r = 0; r < c->batch; ++r) sel[r] = (!c->finished[r] && !c->refreshed[r] && (!mask || mask[r]));
    HIP_TRY(hipEventRecord(c->ev0, c->stream));
    dinfer_status s = dinfer_refresh_kv(c, sel.data());
    if (s != DINFER_OK) return s;
    HIP_TRY(hipEventRecord(c->ev1, c->stream));
    HIP_TRY(hipEventSynchronize(c->ev1));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, c->ev0, c->ev1));
    refresh_ms += ms;
    stats.refreshes += n;
    // expert cache: a block start re-places the experts from the routing of
    // the refresh just run (and of the steps since the last placement)
    return c->offload ? place_experts(c, true) : DINFER_OK;
  };
  dinfer_status s = refresh(nullptr);
  if (s != DINFER_OK) return s;
  const int U = c->dc.graph_unroll;
  while (unfinished(c) > 0) {
    if (stats.steps >= max_steps) return fail(DINFER_E_STATE, "max_steps reached before completion");
    if (c->step_dirty) {
      s = upload_step_table(c);
      if (s != DINFER_OK) return s;
    }
    if (U > 0) {
      if (!c->graph || c->graph_steps != U) {
        s = capture_graph(c, U);
        if (s != DINFER_OK) return s;
      }
      HIP_TRY(hipGraphLaunch(c->graph, c->stream));
      stats.steps += U;
    } else {
      s = dinfer_denoise_step(c);
      if (s == DINFER_OK) s = dinfer_commit(c);
      if (s != DINFER_OK) return s;
      stats.steps += 1;
    }
    if (c->offload && c->interval > 0) {
      c->steps_since_place += U > 0 ? U : 1;
      if (c->steps_since_place >= c->interval) {
        s = place_experts(c, false);
        if (s != DINFER_OK) return s;
      }
    }
    s = dinfer_advance_blocks(c, need.data(), nullptr);
    if (s != DINFER_OK) return s;
    s = refresh(need.data());
    if (s != DINFER_OK) return s;
  }
  std::vector<int> cc(c->batch);
  HIP_TRY(hipMemcpyAsync(cc.data(), c->at<int>(c->L.off_ccount), (size_t)c->batch * 4,
                         hipMemcpyDeviceToHost, c->stream));
  HIP_TRY(hipStreamSynchronize(c->stream));
  for (int r = 0; r < c->batch; ++r) stats.committed += cc[r];
  stats.wall_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
  stats.refresh_ms = refresh_ms;
  if (h_stats) *h_stats = stats;
  return DINFER_OK;
}

size_t dinfer_expert_slot_bytes(const dinfer_model_cfg* m) {
  if (!m || m->n_experts < 1 || m->expert_ffn < 1 || m->d_model < 1) return 0;
  if (m->dtype != DINFER_F32 && m->dtype != DINFER_BF16) return 0;
  return (size_t)3 * m->expert_ffn * m->d_model * (m->dtype == DINFER_F32 ? 4 : 2);
}

dinfer_status dinfer_expert_offload(dinfer_ctx* c, const void* const* h_exp_gate_up,
                                    const void* const* h_exp_down, int32_t slots,
                                    int32_t interval, void* d_slots, size_t slots_bytes) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  const Layout& L = c->L;
  if (!L.moe) return fail(DINFER_E_ARG, "expert offload needs an MoE model");
  if (c->offload) return fail(DINFER_E_STATE, "the expert cache is already configured");
  if (slots < 1 || slots > L.E) return fail(DINFER_E_ARG, "slots must be in 1..n_experts");
  if (interval < 0) return fail(DINFER_E_ARG, "interval must be >= 0");
  if (!h_exp_gate_up || !h_exp_down) return fail(DINFER_E_ARG, "null expert store");
  const size_t one = expert_gu_bytes(L) + expert_dn_bytes(L);
  if (!d_slots) return fail(DINFER_E_WORKSPACE, "slot buffer is null");
  if (reinterpret_cast<uintptr_t>(d_slots) % kAlign != 0)
    return fail(DINFER_E_WORKSPACE, "slot buffer must be 256-byte aligned");
  if (slots_bytes < (size_t)L.nl * slots * one)
    return fail(DINFER_E_WORKSPACE, "slot buffer too small: need " +
                                        std::to_string((size_t)L.nl * slots * one) + " bytes");
  std::vector<const char*> gu(L.nl), dn(L.nl), dgu(L.nl), ddn(L.nl);
  for (int l = 0; l < L.nl; ++l) {
    if (!h_exp_gate_up[l] || !h_exp_down[l]) return fail(DINFER_E_ARG, "null expert store entry");
    void* a = nullptr;
    void* b = nullptr;
    if (hipHostGetDevicePointer(&a, const_cast<void*>(h_exp_gate_up[l]), 0) != hipSuccess ||
        hipHostGetDevicePointer(&b, const_cast<void*>(h_exp_down[l]), 0) != hipSuccess || !a || !b) {
      (void)hipGetLastError();
      return fail(DINFER_E_ARG, "the expert store must be pinned host memory (hipHostMalloc)");
    }
    gu[l] = static_cast<const char*>(h_exp_gate_up[l]);
    dn[l] = static_cast<const char*>(h_exp_down[l]);
    dgu[l] = static_cast<const char*>(a);
    ddn[l] = static_cast<const char*>(b);
  }
  HIP_TRY(hipStreamSynchronize(c->stream));
  c->h_gu = gu;
  c->h_dn = dn;
  c->hd_gu = dgu;
  c->hd_dn = ddn;
  c->d_slots = static_cast<char*>(d_slots);
  c->slots = slots;
  c->interval = interval;
  c->slot_expert.assign(L.nl, std::vector<int>(slots, -1));
  // start with experts 0..slots-1 of every layer in HBM, the rest in the store
  for (int l = 0; l < L.nl; ++l)
    for (int e = 0; e < L.E; ++e) {
      if (e < slots) {
        dinfer_status st = move_expert_in(c, l, e, e);
        if (st != DINFER_OK) return st;
      } else {
        move_expert_out(c, l, e);
      }
    }
  dinfer_status st = upload_expert_tables(c, true);
  if (st != DINFER_OK) return st;
  HIP_TRY(hipMemsetAsync(c->at<char>(L.off_eacct), 0, (size_t)L.nl * 4 * 8, c->stream));
  HIP_TRY(hipStreamSynchronize(c->stream));
  c->offload = true;
  c->experts_ready = true;
  c->steps_since_place = 0;
  if (c->graph) {   // the step now also records expert usage
    (void)hipGraphExecDestroy(c->graph);
    c->graph = nullptr;
    c->graph_steps = 0;
  }
  return DINFER_OK;
}

dinfer_status dinfer_expert_place(dinfer_ctx* c) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  if (!c->offload) return fail(DINFER_E_STATE, "no expert cache (dinfer_expert_offload)");
  return place_experts(c, true);
}

dinfer_status dinfer_expert_cache_report(dinfer_ctx* c, dinfer_expert_cache_stats* out,
                                         int32_t reset) {
  if (!c || !out) return fail(DINFER_E_ARG, "null argument");
  if (!c->offload) return fail(DINFER_E_STATE, "no expert cache (dinfer_expert_offload)");
  const Layout& L = c->L;
  std::vector<long long> a((size_t)L.nl * 4);
  HIP_TRY(hipMemcpyAsync(a.data(), c->at<long long>(L.off_eacct), a.size() * 8,
                         hipMemcpyDeviceToHost, c->stream));
  HIP_TRY(hipStreamSynchronize(c->stream));
  dinfer_expert_cache_stats r{};
  for (int l = 0; l < L.nl; ++l) {
    r.expert_hits += a[(size_t)l * 4 + 0];
    r.expert_misses += a[(size_t)l * 4 + 1];
    r.row_hits += a[(size_t)l * 4 + 2];
    r.row_misses += a[(size_t)l * 4 + 3];
  }
  r.bytes_placed = c->bytes_h2d;
  r.bytes_host_read = r.expert_misses * (int64_t)(expert_gu_bytes(L) + expert_dn_bytes(L));
  r.placements = c->placements;
  r.slots = c->slots;
  r.interval = c->interval;
  *out = r;
  if (reset) {
    HIP_TRY(hipMemsetAsync(c->at<char>(L.off_eacct), 0, (size_t)L.nl * 4 * 8, c->stream));
    c->bytes_h2d = 0;
    c->placements = 0;
  }
  return DINFER_OK;
}

dinfer_status dinfer_set_activation_precision(dinfer_ctx* c, uint32_t step_mask,
                                              uint32_t refresh_mask) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  if ((step_mask | refresh_mask) & ~0x1Fu) return fail(DINFER_E_ARG, "masks hold bits 0..4 only");
  if (c->L.dt != DType::BF16 && (step_mask | refresh_mask))
    return fail(DINFER_E_UNSUPPORTED, "bf16-only activations need bf16 weights");
  if (c->graph && step_mask != c->hi_only_step) {
    (void)hipGraphExecDestroy(c->graph);
    c->graph = nullptr;
    c->graph_steps = 0;
  }
  c->hi_only_step = step_mask;
  c->hi_only_refresh = refresh_mask;
  return DINFER_OK;
}

dinfer_status dinfer_keep_logits(dinfer_ctx* c, int32_t on) {
  if (!c) return fail(DINFER_E_ARG, "ctx is null");
  if ((on != 0) != c->keep_logits && c->graph) {
    // the captured step graph holds the LM head's arguments
    (void)hipGraphExecDestroy(c->graph);
    c->graph = nullptr;
    c->graph_steps = 0;
  }
  c->keep_logits = on != 0;
  return DINFER_OK;
}

dinfer_status dinfer_get_step_view(const dinfer_ctx* c, dinfer_step_view* v) {
  if (!c || !v) return fail(DINFER_E_ARG, "null argument");
  const Layout& L = c->L;
  v->batch = c->batch;
  v->block_len = L.B;
  v->vocab = L.V;
  v->topk = 8;
  v->logits = c->at<float>(L.off_logits);
  v->argmax = c->at<int>(L.off_argmax);
  v->conf = c->at<float>(L.off_conf);
  v->lse = c->at<float>(L.off_lse);
  v->topk_id = c->at<int>(L.off_tid);
  v->topk_p = c->at<float>(L.off_tp);
  v->credit = c->at<float>(L.off_credit);
  v->tracked = c->at<int>(L.off_tracked);
  v->smooth_id = c->at<int>(L.off_sid);
  v->smooth_p = c->at<float>(L.off_sp);
  v->smooth_valid = c->at<uint8_t>(L.off_sv);
  v->commit_mask = c->at<uint8_t>(L.off_cm);
  v->block_done = c->at<int>(L.off_done);
  v->step_count = c->at<int>(L.off_steps);
  v->commit_count = c->at<int>(L.off_ccount);
  v->decode_stats = c->at<int>(L.off_dstat);
  v->decode_stat_words = kDecodeStatWords;
  v->kv_k = c->at<char>(L.off_kvk);
  v->kv_v = c->at<char>(L.off_kvv);
  v->kv_len = L.Lp;
  v->moe_top_k = L.moe ? L.topk : 0;
  v->moe_sel = L.moe ? c->at<int>(L.off_sel) : nullptr;
  v->moe_gate = L.moe ? c->at<float>(L.off_gate) : nullptr;
  v->moe_experts = L.moe ? L.E : 0;
  v->moe_logits = L.moe ? c->at<float>(L.off_rlog) : nullptr;
  v->ffn_in = c->at<float>(L.off_a);
  return DINFER_OK;
}

dinfer_status dinfer_pack_linear(const void* d_W, void* d_packed, int32_t n_mats, int32_t rows,
                                 int32_t K, int32_t dtype, void* stream) {
  if (!d_W || !d_packed) return fail(DINFER_E_ARG, "null pointer");
  if (d_W == d_packed) return fail(DINFER_E_ARG, "packing in place is not supported");
  if (dtype != DINFER_F32 && dtype != DINFER_BF16) return fail(DINFER_E_ARG, "bad dtype");
  const DType dt = dtype == DINFER_F32 ? DType::F32 : DType::BF16;
  const int kstep = dt == DType::F32 ? 16 : 32;
  if (n_mats < 1 || n_mats > 65535) return fail(DINFER_E_ARG, "n_mats must be in 1..65535");
  if (rows < 16 || rows % 16 != 0) return fail(DINFER_E_ARG, "rows must be a positive multiple of 16");
  if (K < kstep || K % kstep != 0) return fail(DINFER_E_ARG, "K must be a positive multiple of 32 (bf16) / 16 (f32)");
  const size_t bytes = (size_t)n_mats * rows * K * dtype_size(dt);
  const char* a = static_cast<const char*>(d_W);
  const char* b = static_cast<const char*>(d_packed);
  if (a < b + bytes && b < a + bytes) return fail(DINFER_E_ARG, "source and destination overlap");
  HIP_TRY(launch_pack_linear(dt, d_W, d_packed, n_mats, rows, K, static_cast<hipStream_t>(stream)));
  return DINFER_OK;
}

size_t dinfer_linear_out_elems(int32_t M, int32_t N, int32_t K, int32_t dtype) {
  if (M < 1 || (dtype != DINFER_F32 && dtype != DINFER_BF16)) return 0;
  const DType dt = dtype == DINFER_F32 ? DType::F32 : DType::BF16;
  if (!gemm_shape_ok(dt, N, K)) return 0;
  const GemmPlan p = plan_gemm(dt, M, N, K, 256);
  return (size_t)p.splits * M * N;
}

dinfer_status dinfer_linear(const float* d_A, const void* d_W, float* d_out, int32_t M, int32_t N,
                            int32_t K, int32_t dtype, int32_t* h_splits, void* stream) {
  if (!d_A || !d_W || !d_out) return fail(DINFER_E_ARG, "null pointer");
  if (M < 1) return fail(DINFER_E_ARG, "M must be positive");
  if (dtype != DINFER_F32 && dtype != DINFER_BF16) return fail(DINFER_E_ARG, "bad dtype");
  const DType dt = dtype == DINFER_F32 ? DType::F32 : DType::BF16;
  if (!gemm_shape_ok(dt, N, K)) return fail(DINFER_E_UNSUPPORTED, "N % 128 or K chunk multiple");
  const GemmPlan p = plan_gemm(dt, M, N, K, 256);
  if (h_splits) *h_splits = p.splits;
  HIP_TRY(launch_gemm(p, dt, d_A, d_W, d_out, nullptr, M, N, K, static_cast<hipStream_t>(stream)));
  return DINFER_OK;
}

size_t dinfer_vocab_stats_scratch_bytes(int32_t rows, int32_t vocab) {
  if (rows < 1 || vocab < 2) return 0;
  return vocab_scratch_bytes(plan_vocab(rows, vocab, 1024), rows);
}

dinfer_status dinfer_vocab_stats(const float* d_logits, int32_t rows, int32_t vocab,
                                 const int32_t* d_plant_id, const float* d_plant_bias,
                                 int32_t mask_id, int32_t* d_argmax, float* d_conf, float* d_lse,
                                 int32_t* d_topk_id, float* d_topk_p, void* d_scratch,
                                 size_t scratch_bytes, void* stream) {
  if (!d_logits || !d_argmax || !d_conf || !d_lse || !d_topk_id || !d_topk_p)
    return fail(DINFER_E_ARG, "null output or input pointer");
  if (rows < 1 || vocab < 2) return fail(DINFER_E_ARG, "rows and vocab must be positive");
  if (vocab % 4 != 0) return fail(DINFER_E_UNSUPPORTED, "vocab must be a multiple of 4");
  if (mask_id < -1 || mask_id >= vocab) return fail(DINFER_E_ARG, "mask_id out of range");
  const VocabPlan p = plan_vocab(rows, vocab, 1024);
  if (!d_scratch || scratch_bytes < vocab_scratch_bytes(p, rows))
    return fail(DINFER_E_WORKSPACE, "scratch too small");
  HIP_TRY(launch_vocab_stats(p, d_logits, rows, vocab, d_plant_id, d_plant_bias, mask_id, d_scratch,
                             d_argmax, d_conf, d_lse, d_topk_id, d_topk_p,
                             static_cast<hipStream_t>(stream)));
  return DINFER_OK;
}

dinfer_status dinfer_vocab_stats_noalloc(const float* d_logits, int32_t rows, int32_t vocab,
                                         const int32_t* d_plant_id, const float* d_plant_bias,
                                         int32_t mask_id, int32_t* d_argmax, float* d_conf,
                                         float* d_lse, int32_t* d_topk_id, float* d_topk_p,
                                         void* stream) {
  if (!d_logits || !d_argmax || !d_conf || !d_lse || !d_topk_id || !d_topk_p)
    return fail(DINFER_E_ARG, "null output or input pointer");
  if (rows < 1 || vocab < 2) return fail(DINFER_E_ARG, "rows and vocab must be positive");
  if (vocab % 4 != 0) return fail(DINFER_E_UNSUPPORTED, "vocab must be a multiple of 4");
  if (mask_id < -1 || mask_id >= vocab) return fail(DINFER_E_ARG, "mask_id out of range");
  const VocabPlan p = plan_vocab(rows, vocab, 1024);
  const size_t need = vocab_scratch_bytes(p, rows);
  if (need > kNoAllocScratchBytes)
    return fail(DINFER_E_UNSUPPORTED,
                "rows x vocab splits need " + std::to_string(need) +
                    " bytes of scratch, above the fixed " +
                    std::to_string(kNoAllocScratchBytes) + " of the no-allocation entry point");
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(DINFER_E_UNSUPPORTED, "device index above 63");
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      // first call on this device (it is current): its copy of the array
      void* a = nullptr;
      HIP_TRY(hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)));
      if (!a) return fail(DINFER_E_HIP, "hipGetSymbolAddress returned no address");
      g_scratch_ptr[dev] = a;
    }
    ptr = g_scratch_ptr[dev];
  }
  HIP_TRY(launch_vocab_stats(p, d_logits, rows, vocab, d_plant_id, d_plant_bias, mask_id, ptr,
                             d_argmax, d_conf, d_lse, d_topk_id, d_topk_p,
                             static_cast<hipStream_t>(stream)));
  return DINFER_OK;
}

void dinfer_destroy(dinfer_ctx* c) {
  if (!c) return;
  if (c->graph) (void)hipGraphExecDestroy(c->graph);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
  if (c->ev_join) (void)hipEventDestroy(c->ev_join);
  if (c->ev_step_upload) (void)hipEventDestroy(c->ev_step_upload);
  if (c->ev_ref_upload) (void)hipEventDestroy(c->ev_ref_upload);
  if (c->ev0) (void)hipEventDestroy(c->ev0);
  if (c->ev1) (void)hipEventDestroy(c->ev1);
  if (c->h_tab_step) (void)hipHostFree(c->h_tab_step);
  if (c->h_tab_ref) (void)hipHostFree(c->h_tab_ref);
  if (c->h_misc) (void)hipHostFree(c->h_misc);
  if (c->h_wtab) (void)hipHostFree(c->h_wtab);
  if (c->h_resident) (void)hipHostFree(c->h_resident);
  delete c;
}

}  // extern "C"
