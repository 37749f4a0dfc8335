// Host side of libspecverify: argument validation, scratch management and
// kernel dispatch for the C ABI declared in include/specverify.h.
#include "sv_common.hpp"
#include "specverify.h"

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <mutex>

namespace sv {
hipError_t launch_stream(const Args& a, int dtype, int mode, bool vec, unsigned grid, hipStream_t s,
                         hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
hipError_t launch_row(const Args& a, int dtype, int mode, unsigned grid, hipStream_t s);
hipError_t launch_sample(const Args& a, int dtype, unsigned grid, hipStream_t s);
hipError_t launch_probs(const Args& a, int dtype, int mode, unsigned grid, hipStream_t s);
hipError_t launch_lm_gemm(const void* H, const void* W, float* C, int32_t M, int32_t V, int32_t d, hipStream_t s);
int64_t lm_gemm_tiles(int32_t M, int32_t V);
}  // namespace sv

using namespace sv;

namespace {

constexpr int kMaxDevices = 64;
// A launch must satisfy grid * WG < 2^32.
constexpr int64_t kMaxGrid = (int64_t(1) << 32) / WG - 1;

struct Scratch {
  char* ptr = nullptr;
  size_t bytes = 0;
  int64_t cap_seq = 0;   // sequences the (zero-filled) arrival counters cover
};

std::mutex g_mu;
Scratch g_scr[kMaxDevices];

// Logits formed by the output projection for verification (float32, target
// rows then draft rows), per device, grown on demand (guarded by g_mu).
struct LogitBuf {
  float* ptr = nullptr;
  size_t bytes = 0;
};
LogitBuf g_lgt[kMaxDevices];

// Launch timing (sv_profile_start / sv_profile_stop): three events per call:
// the streaming kernel's start and end (recorded by its launch), and one
// recorded on the call's stream after the call's last kernel.  Slots are
// reused round-robin; a slot is folded into the totals (synchronising on its
// last event) before reuse.
constexpr int kProfSlots = 1024;
struct ProfSlot {
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  bool pending = false;
};
struct Profile {
  bool on = false;
  int next = 0;
  double stream_ms = 0.0, rest_ms = 0.0;
  int64_t calls = 0;
  ProfSlot slot[kProfSlots];
};
std::mutex g_prof_mu;
Profile g_prof;

// Folds a recorded slot into the totals (caller holds g_prof_mu).
int prof_fold(ProfSlot& sl) {
  if (!sl.pending) return SV_OK;
  sl.pending = false;
  float a = 0.f, b = 0.f;
  if (hipEventSynchronize(sl.ev[2]) != hipSuccess || hipEventElapsedTime(&a, sl.ev[0], sl.ev[1]) != hipSuccess ||
      hipEventElapsedTime(&b, sl.ev[1], sl.ev[2]) != hipSuccess)
    return SV_ERR_HIP;
  g_prof.stream_ms += a;
  g_prof.rest_ms += b;
  g_prof.calls += 1;
  return SV_OK;
}

// Takes the next slot for a call (nullptr when timing is off).
ProfSlot* prof_begin() {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof.on) return nullptr;
  ProfSlot& sl = g_prof.slot[g_prof.next];
  g_prof.next = (g_prof.next + 1) % kProfSlots;
  if (prof_fold(sl) != SV_OK) return nullptr;
  // timing only: no system-scope fence (cache writeback and invalidation)
  // when an event is reached, which would add to the measured launches
  for (hipEvent_t& e : sl.ev)
    if (!e && hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return &sl;
}

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t seq_cnt, smp_cnt, chunk, ctop, cand, row, kidx, kprob, seq, seg_sum, seg_last, qxs, total;
};

// What one call needs from the scratch.
struct Need {
  int64_t rows = 0, nchunks = 0, B = 0, nseg = 0;  // nseg: sampling segments per sequence
  bool filt = false;                               // candidate and kept lists
  bool topk = false;                               // the chunks' largest thread maxima
};

// Counters first (a fixed region for the life of the allocation: the kernels
// leave every counter at zero, so it never needs clearing), then the data
// records of the call.
Layout make_layout(int64_t cap_seq, const Need& n) {
  Layout L;
  size_t o = 0;
  L.seq_cnt = o; o += al256(cap_seq * 4);
  L.smp_cnt = o; o += al256(cap_seq * 4);
  L.chunk = o; o += al256(n.rows * n.nchunks * sizeof(ChunkRec));
  L.ctop = o; o += n.topk ? al256(n.rows * n.nchunks * CTOP * sizeof(uint32_t)) : 0;
  L.cand = o; o += n.filt ? al256(n.rows * n.nchunks * CAND_CAP * sizeof(uint64_t)) : 0;
  L.row = o; o += al256(n.rows * sizeof(RowRec));
  L.kidx = o; o += n.filt ? al256(n.rows * KEEP_CAP * sizeof(int32_t)) : 0;
  L.kprob = o; o += n.filt ? al256(n.rows * KEEP_CAP * sizeof(double)) : 0;
  L.seq = o; o += al256(n.B * sizeof(SeqRec));
  L.seg_sum = o; o += al256(n.B * n.nseg * sizeof(double));
  L.seg_last = o; o += al256(n.B * n.nseg * sizeof(int32_t));
  L.qxs = o; o += al256(n.rows * sizeof(float));
  L.total = o;
  return L;
}

// Returns the scratch of the current device, large enough for this call.
int get_scratch(const Need& n, char** base, Layout* lay) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  Scratch& s = g_scr[dev];
  Layout L = make_layout(s.cap_seq, n);
  if (s.ptr == nullptr || s.cap_seq < n.B || s.bytes < L.total) {
    const int64_t cs = std::max(n.B, s.cap_seq);
    L = make_layout(cs, n);
    const size_t want = std::max(L.total, s.bytes);
    if (s.ptr) {
      if (hipDeviceSynchronize() != hipSuccess) return SV_ERR_HIP;
      (void)hipFree(s.ptr);
      s.ptr = nullptr;
      s.bytes = 0;
      s.cap_seq = 0;
    }
    void* p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) return SV_ERR_WORKSPACE;
    if (hipMemset(p, 0, want) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
      (void)hipFree(p);
      return SV_ERR_HIP;
    }
    s.ptr = (char*)p;
    s.bytes = want;
    s.cap_seq = cs;
  }
  *base = s.ptr;
  *lay = make_layout(s.cap_seq, n);
  return SV_OK;
}

void bind_scratch(Args& a, char* base, const Layout& L) {
  a.seq_cnt = (uint32_t*)(base + L.seq_cnt);
  a.smp_cnt = (uint32_t*)(base + L.smp_cnt);
  a.chunk = (ChunkRec*)(base + L.chunk);
  a.ctop = (uint32_t*)(base + L.ctop);
  a.cand = (uint64_t*)(base + L.cand);
  a.row = (RowRec*)(base + L.row);
  a.kidx = (int32_t*)(base + L.kidx);
  a.kprob = (double*)(base + L.kprob);
  a.seq = (SeqRec*)(base + L.seq);
  a.seg_sum = (double*)(base + L.seg_sum);
  a.seg_last = (int32_t*)(base + L.seg_last);
  a.qxs = (float*)(base + L.qxs);
}

int check_params(float T, int32_t top_k, float top_p) {
  if (!(T >= 0.0f) || !std::isfinite(T) || (T > 0.0f && T < FLT_MIN)) return SV_ERR_PARAM;
  if (top_k < 0) return SV_ERR_PARAM;
  if (!(top_p > 0.0f && top_p <= 1.0f)) return SV_ERR_PARAM;
  return SV_OK;
}

int pick_mode(float T, int32_t top_k, float top_p, int32_t V) {
  if (T == 0.0f) return M_GREEDY;
  const bool k = top_k > 0 && top_k < V;
  const bool p = top_p < 1.0f;
  return k && p ? M_TOPKP : k ? M_TOPK : p ? M_TOPP : M_PLAIN;
}

void temp_scalars(float T, float* c2, float* win, double* invT) {
  if (T > 0.0f) {
    *invT = 1.0 / (double)T;
    *c2 = (float)(1.4426950408889634074 / (double)T);
    *win = TOPP_WINDOW_Z * T;
  } else {
    *invT = 0.0;
    *c2 = 0.0f;
    *win = 0.0f;
  }
}

// Td: the draft rows' temperature (the target's unless the drafts were
// sampled at another one).
void set_scalars(Args& a, float T, int32_t top_k, float top_p, float Td) {
  a.top_k = top_k;
  a.top_p = (double)top_p;
  temp_scalars(T, &a.c2, &a.win, &a.invT);
  temp_scalars(T > 0.0f ? Td : T, &a.c2d, &a.wind, &a.invTd);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A ragged batch: per-sequence draft counts from device offsets cu[B + 1]
// (nd drafts in total, at most kmax per sequence).
struct Ragged {
  const int32_t* cu;
  int32_t nd, kmax;
};

// need_n: out_n is required (the sampler passes none).  out_px: probability
// of each sequence's last drawn token under the row it was drawn from (the
// sampler, K == 0).  rg: null for a rectangular [B, K] batch.  qprob: the
// draft distributions given as probabilities [B, K, V] (rectangular only;
// drf is then not used).
int verify_impl(const void* tgt, const void* drf, const int32_t* X, const float* U, float T, float Td,
                int32_t top_k, float top_p, int32_t* out_tok, int32_t* out_n, bool need_n, double* out_p,
                double* out_q, double* out_z, double* out_px, int32_t B, int32_t K, int32_t V, int32_t dtype,
                void* stream, const Ragged* rg = nullptr, const float* qprob = nullptr, bool qp = false,
                bool timed = true) {
  if (B < 0 || K < 0 || K > SV_MAX_K || V < 1 || V > MAX_V) return SV_ERR_SHAPE;
  if (rg && (rg->nd < 0 || rg->kmax < 0 || rg->kmax > SV_MAX_K || (int64_t)rg->nd > (int64_t)B * rg->kmax))
    return SV_ERR_SHAPE;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  int st = check_params(T, top_k, top_p);
  if (st != SV_OK) return st;
  // at T > 0 the draft temperature must be a valid temperature above 0
  if (T > 0.0f && (check_params(Td, top_k, top_p) != SV_OK || !(Td > 0.0f))) return SV_ERR_PARAM;
  if (B == 0) return SV_OK;
  const int mode = pick_mode(T, top_k, top_p, V);
  const int64_t nd = rg ? rg->nd : (int64_t)B * K;  // draft rows
  const int32_t kmax = rg ? rg->kmax : K;
  if (!tgt || !U || !out_tok || (need_n && !out_n) || (rg && !rg->cu)) return SV_ERR_NULL;
  if (nd > 0 && !X) return SV_ERR_NULL;
  if (nd > 0 && mode != M_GREEDY && !(qp ? (const void*)qprob : drf)) return SV_ERR_NULL;
  // q given as probabilities: no draft rows to stream (greedy never uses q)
  const bool use_qp = qp && mode != M_GREEDY && nd > 0;
  const int esz = dtype == SV_BF16 ? 2 : 4;
  const int64_t nt = nd + B;  // target rows
  const int64_t rows = (mode == M_GREEDY || use_qp) ? nt : nt + nd;
  const int64_t nchunks = ((int64_t)V + CE - 1) / CE;
  const int64_t nsc = ((int64_t)V + SCE - 1) / SCE;
  if (rows * nchunks > kMaxGrid || (int64_t)B * nsc > kMaxGrid) return SV_ERR_SHAPE;
  Need need;
  need.rows = rows;
  need.nchunks = nchunks;
  need.B = B;
  need.nseg = nsc * SEG_PER_SCE;
  need.filt = mode == M_TOPK || mode == M_TOPP || mode == M_TOPKP;
  need.topk = mode == M_TOPK || mode == M_TOPKP;

  char* base = nullptr;
  Layout L;
  st = get_scratch(need, &base, &L);
  if (st != SV_OK) return st;

  Args a;
  a.tgt = tgt;
  a.drf = (mode == M_GREEDY || use_qp) ? nullptr : drf;
  a.qprob = use_qp ? qprob : nullptr;
  a.X = X;
  a.U = U;
  a.out_tok = out_tok;
  a.out_n = out_n;
  a.out_p = out_p;
  a.out_q = out_q;
  a.out_z = out_z;
  a.out_px = out_px;
  a.out_probs = nullptr;
  a.B = B;
  a.K = rg ? 0 : K;
  a.V = V;
  a.NT = (int32_t)nt;
  a.ND = (int32_t)nd;
  a.Kmax = kmax;
  a.cu = rg ? rg->cu : nullptr;
  a.nchunks = (int32_t)nchunks;
  a.nsc = (int32_t)nsc;
  // sampling chunks per workgroup: up to SPW (fewer, longer workgroups
  // measured faster), while at least one workgroup per compute unit remains
  a.spw = (int32_t)std::max<int64_t>(1, std::min<int64_t>(SPW, (int64_t)B * nsc / 256));
  a.nsw = (int32_t)((nsc + a.spw - 1) / a.spw);
  a.do_seq = 1;
  set_scalars(a, T, top_k, top_p, Td);
  bind_scratch(a, base, L);

  const bool vec = aligned16(tgt) && (a.drf == nullptr || aligned16(a.drf)) && ((int64_t)V * esz) % 16 == 0;
  a.ulen = vec ? 16 / esz : 1;
  a.dch = make_udiv((uint32_t)a.nchunks);
  a.rps = rg ? 1 : (mode == M_GREEDY || use_qp) ? a.K + 1 : 2 * a.K + 1;
  a.drps = make_udiv((uint32_t)a.rps);
  hipStream_t s = (hipStream_t)stream;
  ProfSlot* prof = timed ? prof_begin() : nullptr;
  // chunk-parallel streaming pass, then one workgroup per row merges it; the
  // last row of each sequence finishes the sequence.  When timing, the
  // streaming launch records its own start and end in the slot's events.
  if (launch_stream(a, dtype, mode, vec, (unsigned)(rows * nchunks), s, prof ? prof->ev[0] : nullptr,
                    prof ? prof->ev[1] : nullptr) != hipSuccess)
    return SV_ERR_HIP;
  if (launch_row(a, dtype, mode, (unsigned)rows, s) != hipSuccess) return SV_ERR_HIP;
  if (mode == M_PLAIN) {
    if (launch_sample(a, dtype, (unsigned)((int64_t)B * a.nsw), s) != hipSuccess) return SV_ERR_HIP;
  }
  if (prof) {
    if (hipEventRecord(prof->ev[2], s) != hipSuccess) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    prof->pending = true;
  }
  return SV_OK;
}

// Largest hidden width accepted (the kernel needs only d % 64 == 0).
constexpr int32_t kMaxHidden = 1 << 16;

int check_lm_shape(const void* H, const void* W, int64_t M, int32_t V, int32_t d) {
  if (M < 0 || V < 1 || V > MAX_V || d < 64 || d > kMaxHidden || d % 64 != 0) return SV_ERR_SHAPE;
  if (M > 0 && (!H || !W)) return SV_ERR_NULL;
  if (M > 0 && (!aligned16(H) || !aligned16(W))) return SV_ERR_SHAPE;
  if (M > INT32_MAX || sv::lm_gemm_tiles((int32_t)std::min<int64_t>(M, INT32_MAX), V) > kMaxGrid) return SV_ERR_SHAPE;
  return SV_OK;
}

// The logits buffer of the current device, at least `bytes` long.
int get_logit_buf(size_t bytes, float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  LogitBuf& b = g_lgt[dev];
  if (b.bytes < bytes) {
    if (b.ptr) {
      if (hipDeviceSynchronize() != hipSuccess) return SV_ERR_HIP;
      (void)hipFree(b.ptr);
      b = LogitBuf();
    }
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) return SV_ERR_WORKSPACE;
    b.ptr = (float*)p;
    b.bytes = bytes;
  }
  *out = b.ptr;
  return SV_OK;
}

}  // namespace

extern "C" {

int sv_lm_logits(const void* hidden, const void* weight, float* out_logits, int32_t M, int32_t V, int32_t d,
                 void* stream) {
  int st = check_lm_shape(hidden, weight, M, V, d);
  if (st != SV_OK) return st;
  if (M == 0) return SV_OK;
  if (!out_logits) return SV_ERR_NULL;
  return launch_lm_gemm(hidden, weight, out_logits, M, V, d, (hipStream_t)stream) == hipSuccess ? SV_OK
                                                                                                : SV_ERR_HIP;
}

int sv_spec_verify_lmhead(const void* hidden_target, const void* weight_target, const void* hidden_draft,
                          const void* weight_draft, const int32_t* draft_tokens, const float* uniforms,
                          float temperature, int32_t top_k, float top_p, int32_t* out_tokens,
                          int32_t* out_num_accepted, double* out_p, double* out_q, double* out_z, int32_t B,
                          int32_t K, int32_t V, int32_t d_target, int32_t d_draft, void* stream) {
  if (B < 0 || K < 0 || K > SV_MAX_K) return SV_ERR_SHAPE;
  int st = check_params(temperature, top_k, top_p);
  if (st != SV_OK) return st;
  const bool greedy = temperature == 0.0f;
  const int64_t mt = (int64_t)B * (K + 1), md = greedy ? 0 : (int64_t)B * K;
  st = check_lm_shape(hidden_target, weight_target, mt, V, d_target);
  if (st != SV_OK) return st;
  if (md > 0 && (st = check_lm_shape(hidden_draft, weight_draft, md, V, d_draft)) != SV_OK) return st;
  if (B == 0) return SV_OK;
  if (!uniforms || !out_tokens || !out_num_accepted || (K > 0 && !draft_tokens)) return SV_ERR_NULL;
  float* lg = nullptr;
  st = get_logit_buf((size_t)(mt + md) * (size_t)V * sizeof(float), &lg);
  if (st != SV_OK) return st;
  float* lt = lg;
  float* ld = md > 0 ? lg + (size_t)mt * V : nullptr;
  hipStream_t s = (hipStream_t)stream;
  // when timing, the slot's first two events bracket the two projections and
  // the third follows the verification
  ProfSlot* prof = prof_begin();
  if (prof && hipEventRecord(prof->ev[0], s) != hipSuccess) return SV_ERR_HIP;
  if (launch_lm_gemm(hidden_target, weight_target, lt, (int32_t)mt, V, d_target, s) != hipSuccess) return SV_ERR_HIP;
  if (md > 0 && launch_lm_gemm(hidden_draft, weight_draft, ld, (int32_t)md, V, d_draft, s) != hipSuccess)
    return SV_ERR_HIP;
  if (prof && hipEventRecord(prof->ev[1], s) != hipSuccess) return SV_ERR_HIP;
  st = verify_impl(lt, ld, draft_tokens, uniforms, temperature, temperature, top_k, top_p, out_tokens,
                   out_num_accepted, true, out_p, out_q, out_z, nullptr, B, K, V, SV_F32, stream, nullptr, nullptr,
                   false, false);
  if (st != SV_OK) return st;
  if (prof) {
    if (hipEventRecord(prof->ev[2], s) != hipSuccess) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    prof->pending = true;
  }
  return SV_OK;
}

int sv_spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                   const float* uniforms, float temperature, int32_t top_k, float top_p, int32_t* out_tokens,
                   int32_t* out_num_accepted, int32_t B, int32_t K, int32_t V, int32_t dtype, void* stream) {
  return verify_impl(target_logits, draft_logits, draft_tokens, uniforms, temperature, temperature, top_k, top_p,
                     out_tokens, out_num_accepted, true, nullptr, nullptr, nullptr, nullptr, B, K, V, dtype, stream);
}

int sv_spec_verify_debug(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                         const float* uniforms, float temperature, int32_t top_k, float top_p,
                         int32_t* out_tokens, int32_t* out_num_accepted, double* out_p, double* out_q,
                         double* out_z, int32_t B, int32_t K, int32_t V, int32_t dtype, void* stream) {
  return verify_impl(target_logits, draft_logits, draft_tokens, uniforms, temperature, temperature, top_k, top_p,
                     out_tokens, out_num_accepted, true, out_p, out_q, out_z, nullptr, B, K, V, dtype, stream);
}

int sv_spec_verify_dt(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                      const float* uniforms, float temperature, float draft_temperature, int32_t top_k, float top_p,
                      int32_t* out_tokens, int32_t* out_num_accepted, double* out_p, double* out_q, double* out_z,
                      int32_t B, int32_t K, int32_t V, int32_t dtype, void* stream) {
  return verify_impl(target_logits, draft_logits, draft_tokens, uniforms, temperature, draft_temperature, top_k,
                     top_p, out_tokens, out_num_accepted, true, out_p, out_q, out_z, nullptr, B, K, V, dtype, stream);
}

int sv_spec_verify_ragged(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                          const float* uniforms, const int32_t* cu_num_draft, float temperature,
                          float draft_temperature, int32_t top_k, float top_p, int32_t* out_tokens,
                          int32_t* out_num_accepted, double* out_p, double* out_q, double* out_z, int32_t B,
                          int32_t total_draft, int32_t max_k, int32_t V, int32_t dtype, void* stream) {
  const Ragged rg{cu_num_draft, total_draft, max_k};
  return verify_impl(target_logits, draft_logits, draft_tokens, uniforms, temperature, draft_temperature, top_k,
                     top_p, out_tokens, out_num_accepted, true, out_p, out_q, out_z, nullptr, B, 0, V, dtype, stream,
                     &rg);
}

int sv_spec_verify_probs(const void* target_logits, const float* draft_probs, const int32_t* draft_tokens,
                         const float* uniforms, float temperature, int32_t top_k, float top_p, int32_t* out_tokens,
                         int32_t* out_num_accepted, double* out_p, double* out_q, double* out_z, int32_t B, int32_t K,
                         int32_t V, int32_t dtype, void* stream) {
  return verify_impl(target_logits, nullptr, draft_tokens, uniforms, temperature, temperature, top_k, top_p,
                     out_tokens, out_num_accepted, true, out_p, out_q, out_z, nullptr, B, K, V, dtype, stream,
                     nullptr, draft_probs, true);
}

// The draw of a verification with no drafts: each row is a sequence of one
// position whose only token is drawn from its own filtered distribution with
// its own uniform.
int sv_sample(const void* logits, const float* uniforms, float temperature, int32_t top_k, float top_p,
              int32_t* out_tokens, double* out_prob, int32_t rows, int32_t V, int32_t dtype, void* stream) {
  return verify_impl(logits, nullptr, nullptr, uniforms, temperature, temperature, top_k, top_p, out_tokens, nullptr,
                     false, nullptr, nullptr, nullptr, out_prob, rows, 0, V, dtype, stream);
}

int sv_filtered_probs(const void* logits, int32_t rows, int32_t V, int32_t dtype, float temperature, int32_t top_k,
                      float top_p, float* out_probs, void* stream) {
  if (rows < 0 || V < 1 || V > MAX_V) return SV_ERR_SHAPE;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  int st = check_params(temperature, top_k, top_p);
  if (st != SV_OK) return st;
  if (temperature == 0.0f) return SV_ERR_PARAM;
  if (rows == 0) return SV_OK;
  if (!logits || !out_probs) return SV_ERR_NULL;
  const int mode = pick_mode(temperature, top_k, top_p, V);
  const int esz = dtype == SV_BF16 ? 2 : 4;
  const int64_t nchunks = ((int64_t)V + CE - 1) / CE;
  const int64_t nsc = ((int64_t)V + SCE - 1) / SCE;
  if ((int64_t)rows * nchunks > kMaxGrid || (int64_t)rows * nsc > kMaxGrid) return SV_ERR_SHAPE;
  Need need;
  need.rows = rows;
  need.nchunks = nchunks;
  need.B = rows;
  need.filt = mode != M_PLAIN;
  need.topk = mode == M_TOPK || mode == M_TOPKP;

  char* base = nullptr;
  Layout L;
  st = get_scratch(need, &base, &L);
  if (st != SV_OK) return st;
  Args a = {};
  a.tgt = logits;
  a.out_probs = out_probs;
  a.B = rows;
  a.K = 0;
  a.V = V;
  a.NT = rows;
  a.nchunks = (int32_t)nchunks;
  a.nsc = (int32_t)nsc;
  a.do_seq = 0;
  set_scalars(a, temperature, top_k, top_p, temperature);
  bind_scratch(a, base, L);
  const bool vec = aligned16(logits) && ((int64_t)V * esz) % 16 == 0;
  a.ulen = vec ? 16 / esz : 1;
  a.dch = make_udiv((uint32_t)a.nchunks);
  a.rps = 1;
  a.drps = make_udiv(1u);
  hipStream_t s = (hipStream_t)stream;
  if (launch_stream(a, dtype, mode, vec, (unsigned)((int64_t)rows * nchunks), s) != hipSuccess) return SV_ERR_HIP;
  if (launch_row(a, dtype, mode, (unsigned)rows, s) != hipSuccess) return SV_ERR_HIP;
  if (launch_probs(a, dtype, mode, (unsigned)((int64_t)rows * nsc), s) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

int sv_profile_start(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (ProfSlot& sl : g_prof.slot) sl.pending = false;
  g_prof.on = true;
  g_prof.next = 0;
  g_prof.stream_ms = g_prof.rest_ms = 0.0;
  g_prof.calls = 0;
  return SV_OK;
}

int sv_profile_stop(double* stream_kernel_ms, double* other_kernels_ms, int64_t* calls) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.on = false;
  int rc = SV_OK;
  for (int i = 0; i < kProfSlots; ++i) {
    ProfSlot& sl = g_prof.slot[(g_prof.next + i) % kProfSlots];
    if (prof_fold(sl) != SV_OK) rc = SV_ERR_HIP;
  }
  if (stream_kernel_ms) *stream_kernel_ms = g_prof.stream_ms;
  if (other_kernels_ms) *other_kernels_ms = g_prof.rest_ms;
  if (calls) *calls = g_prof.calls;
  return rc;
}

int sv_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  int rc = SV_OK;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return SV_ERR_HIP;
  for (int d = 0; d < kMaxDevices; ++d) {
    Scratch& s = g_scr[d];
    LogitBuf& b = g_lgt[d];
    if (!s.ptr && !b.ptr) continue;
    if (hipSetDevice(d) != hipSuccess || hipDeviceSynchronize() != hipSuccess) rc = SV_ERR_HIP;
    if (s.ptr && hipFree(s.ptr) != hipSuccess) rc = SV_ERR_HIP;
    if (b.ptr && hipFree(b.ptr) != hipSuccess) rc = SV_ERR_HIP;
    s = Scratch();
    b = LogitBuf();
  }
  (void)hipSetDevice(cur);
  return rc;
}

int64_t sv_scratch_bytes(int device) {
  if (device < 0 || device >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lk(g_mu);
  return (int64_t)(g_scr[device].bytes + g_lgt[device].bytes);
}

const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_NULL: return "SV_ERR_NULL: a required pointer is NULL";
    case SV_ERR_SHAPE: return "SV_ERR_SHAPE: B, K or V out of range";
    case SV_ERR_DTYPE: return "SV_ERR_DTYPE: unknown logit dtype";
    case SV_ERR_PARAM: return "SV_ERR_PARAM: temperature, top_k or top_p out of range";
    case SV_ERR_HIP: return "SV_ERR_HIP: a HIP runtime call failed";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE: scratch allocation failed";
    default: return "unknown status";
  }
}

int sv_version(void) { return 100; }

}  // extern "C"
