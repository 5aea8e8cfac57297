// Parallel-decode commit of one step (dInfer news article, section
// "解码的艺术"; classic top-1 decoding from the section on the three
// bottlenecks): one wave64 per request, lane j = block offset j.
//
//   credit  : every still-masked position, c <- (argmax == tracked ? gamma*c : 0)
//             + lambda*p with one fp32 rounding per operation, tracked <- argmax
//   candidates: all masked positions, or with the hierarchical order the
//             midpoints lo + (hi-lo-1)/2 of the maximal masked runs [lo, hi)
//             of the block (found from the wave's ballot of masked lanes)
//   gate    : commit every candidate with p >= tau or c >= kappa; if none
//             passes, the candidate of highest p (lowest offset on ties)
//   smoothing: each position still masked afterwards keeps its top-8 ids with
//             probabilities renormalised to sum 1 for the next step's soft
//             embedding
//   end-of-sequence (optional): a committed EOS fixes every still-masked
//             response position after it to EOS (dInfer news article, section
//             "系统级压榨": computation after EOS is skipped)
//   block_done: 1 when no MASK remains in the block, 2 when none remains in
//             the whole response either (the request is complete)
//   accounting: per request, commits through the threshold gate, through the
//             credit gate alone, through the fallback, steps that found the
//             block already done (a graph replays steps past a block's end),
//             and a histogram of commits per step (statistics only)
#include "common.h"
#include "kernels.h"

namespace dinfer {

namespace {

__global__ __launch_bounds__(64) void commit_kernel(CommitArgs a) {
  const int r = blockIdx.x;
  const int j = threadIdx.x;
  const int B = a.B;
  const int row = r * B + j;
  const bool inb = j < B;
  int* acct = a.decode_stats + (size_t)r * kDecodeStatWords;
  if (!a.req_active[r] || a.block_done[r]) {
    if (inb) a.commit_mask[row] = 0;
    if (j == 0 && a.req_active[r]) acct[3] += 1;    // idle step: the block is done
    return;
  }
  const int bs = a.req_bs[r];
  int* tok = a.tokens + (size_t)r * a.max_len + bs;
  const bool masked = inb && tok[j] == a.mask_id;
  const int am = inb ? a.argmax[row] : 0;
  const float p = inb ? a.conf[row] : 0.f;
  float c = inb ? a.credit[row] : 0.f;
  if (masked) {
    const float keep = (am == a.tracked[row]) ? __fmul_rn(a.gamma, c) : 0.f;
    c = __fadd_rn(keep, __fmul_rn(a.lambda, p));
    a.credit[row] = c;
    a.tracked[row] = am;
  }

  const unsigned long long mb = __ballot(masked);
  bool cand = masked;
  if (a.hierarchical && masked) {
    // run containing j: lo = one past the highest unmasked offset below j,
    // hi = the lowest unmasked offset above j (offsets >= B count as unmasked)
    const unsigned long long below = (~mb) & ((1ull << j) - 1ull);
    const int lo = below ? 64 - __clzll(below) : 0;
    const unsigned long long above = (j == 63) ? 0ull : ((~mb) & ~((2ull << j) - 1ull));
    int hi = above ? __ffsll((long long)above) - 1 : 64;
    if (hi > B) hi = B;
    cand = (j == lo + (hi - lo - 1) / 2);
  }
  const bool pass = cand && (p >= a.tau || c >= a.kappa);
  const unsigned long long pb = __ballot(pass);
  bool commit = pass;
  if (pb == 0ull) {
    // fallback: highest p among candidates, lowest offset on ties
    float bv = cand ? p : -1.f;
    int bj = cand ? j : 64;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oj = __shfl_xor(bj, o, 64);
      if (ov > bv || (ov == bv && oj < bj)) {
        bv = ov;
        bj = oj;
      }
    }
    commit = cand && j == bj;
  }
  if (commit) tok[j] = am;
  if (inb) a.commit_mask[row] = commit ? 1 : 0;
  // end-of-sequence (early stop): a committed EOS at p fixes every
  // still-masked response position after p to EOS -- the block's lanes here,
  // the positions past the block by the wave's loop.  There is no EOS below
  // the lowest one committed now (a masked position after an earlier EOS
  // would have been filled), so p is the response's first EOS.
  unsigned long long eb = 0ull;
  bool filled = false;
  if (a.eos_id >= 0) {
    eb = __ballot(commit && am == a.eos_id);
    if (eb != 0ull) {
      const int p = __ffsll((long long)eb) - 1;   // block offset
      filled = masked && !commit && j > p;
      if (filled) tok[j] = a.eos_id;
      int* full = a.tokens + (size_t)r * a.max_len;
      for (int i = bs + B + j; i < a.req_len[r]; i += 64)
        if (full[i] == a.mask_id) full[i] = a.eos_id;
    }
  }
  const bool still = masked && !commit && !filled;
  if (inb) {
    if (still) {
      const float* tp = a.topk_p + (size_t)row * 8;
      const int* ti = a.topk_id + (size_t)row * 8;
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) s += tp[k];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        a.smooth_id[(size_t)row * 8 + k] = ti[k];
        a.smooth_p[(size_t)row * 8 + k] = tp[k] / s;
      }
    }
    a.smooth_valid[row] = still ? 1 : 0;
  }
  const unsigned long long sb = __ballot(still);
  const unsigned long long cb = __ballot(commit);
  // with an EOS id, a finished block also finishes the request when no masked
  // response position is left after it (2 = request complete): certainly if
  // this step committed an EOS, else by a scan of the positions past the block
  bool complete = false;
  if (a.eos_id >= 0 && sb == 0ull) {
    if (eb != 0ull) {
      complete = true;
    } else {
      const int* full = a.tokens + (size_t)r * a.max_len;
      bool left = false;
      for (int i = bs + B + j; i < a.req_len[r]; i += 64) left = left || full[i] == a.mask_id;
      complete = !__any(left);
    }
  }
  const int n_tau = __popcll(__ballot(commit && pb != 0ull && p >= a.tau));
  if (j == 0) {
    const int n = __popcll(cb);
    a.step_count[r] += 1;
    a.commit_count[r] += n;
    if (sb == 0ull) a.block_done[r] = complete ? 2 : 1;
    if (pb != 0ull) {
      acct[0] += n_tau;
      acct[1] += n - n_tau;
    } else {
      acct[2] += n;
    }
    acct[4 + n] += 1;
  }
}

// Block start for the selected requests: clear credit, tracked ids,
// smoothing state and the done flag.
__global__ __launch_bounds__(64) void block_reset_kernel(int B, const int* __restrict__ req_mask,
                                                         float* credit, int* tracked,
                                                         uint8_t* smooth_valid,
                                                         uint8_t* commit_mask, int* block_done,
                                                         int* step_count) {
  const int r = blockIdx.x;
  const int j = threadIdx.x;
  if (!req_mask[r]) return;
  if (j < B) {
    credit[r * B + j] = 0.f;
    tracked[r * B + j] = -1;
    smooth_valid[r * B + j] = 0;
    commit_mask[r * B + j] = 0;
  }
  if (j == 0) {
    block_done[r] = 0;
    step_count[r] = 0;
  }
}

// Head of a denoising step: requests whose block is already done take no
// part (their row count in the step table goes to 0, so the attention skips
// them), and when no request has an open block the step's row counts go to
// 0, so every kernel of the step exits at once.  Such steps arise when a
// captured graph of several steps runs past a block's end.  The host writes
// the table afresh whenever blocks move (dinfer_advance_blocks), which
// restores the counts.
__global__ __launch_bounds__(64) void step_gate_kernel(int batch, int* nrows, int* lm_rows,
                                                       int* req_nrows,
                                                       const int* __restrict__ req_active,
                                                       const int* __restrict__ block_done) {
  bool open = false;
  for (int r = threadIdx.x; r < batch; r += 64) {
    const bool act = req_active[r] != 0;
    const bool done = block_done[r] != 0;
    if (act && done) req_nrows[r] = 0;
    open = open || (act && !done);
  }
  if (!__any(open) && threadIdx.x == 0) {
    *nrows = 0;
    *lm_rows = 0;
  }
}

}  // namespace

hipError_t launch_step_gate(int batch, int* nrows, int* lm_rows, int* req_nrows,
                            const int* req_active, const int* block_done, hipStream_t st) {
  hipLaunchKernelGGL(step_gate_kernel, dim3(1), dim3(64), 0, st, batch, nrows, lm_rows, req_nrows,
                     req_active, block_done);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t st) {
  if (a.B > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(commit_kernel, dim3(a.batch), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_block_reset(int batch, int B, const int* req_mask, float* credit, int* tracked,
                              uint8_t* smooth_valid, uint8_t* commit_mask, int* block_done,
                              int* step_count, hipStream_t st) {
  hipLaunchKernelGGL(block_reset_kernel, dim3(batch), dim3(64), 0, st, B, req_mask, credit,
                     tracked, smooth_valid, commit_mask, block_done, step_count);
  return hipGetLastError();
}

}  // namespace dinfer
